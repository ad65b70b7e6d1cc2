"""Helpers for the GPU parity tests: move seeded inputs to the device, run the
HIP path through the C ABI, and compare with the oracle at the tolerance the
method is held to (max |out - ref| <= 1e-2, max |lse - ref| <= 1e-3)."""
import numpy as np

OUT_TOL = 1e-2
LSE_TOL = 1e-3


def to_device(inp, kv_override=None):
    import torch
    dev = torch.device("cuda", 0)

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    return dict(q=bf16(inp.q), kv=bf16(inp.kv_cache if kv_override is None else kv_override),
                bt=torch.from_numpy(inp.block_table).to(dev),
                sl=torch.from_numpy(inp.cache_seqlens).to(dev))


def run_gpu(inp, force_splits=0, num_cus=0, dev_inputs=None, repeat=1, causal=False):
    import torch
    import decode_attention_mla_amd as mla
    d = dev_inputs or to_device(inp)
    sched, ns = mla.get_mla_metadata(inp.cache_seqlens, inp.h_q, inp.s_q, num_cus=num_cus,
                                     force_splits=force_splits)
    out = lse = None
    for _ in range(repeat):
        out, lse = mla.mla_decode_fwd(d["q"], d["kv"], d["bt"], d["sl"], inp.softmax_scale, sched, ns,
                                      causal=causal)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


# Unit roundoff of round-to-nearest-even: bf16 keeps 8 significant bits
# (7 stored + the implicit one), fp32 keeps 24.
U_BF16 = 2.0 ** -8
U_F32 = 2.0 ** -24


def row_out_bound(qrows, keys, scale):
    """Elementwise bound on |out_gpu - out_oracle| for query rows ``qrows``
    (float64 [R, 576]) over the keys they see (float64 [n, 576]), from the
    arithmetic of the HIP path (bf16 inputs, fp32 accumulation):

    * P is rounded to bf16 for the PV product while the row sum keeps fp32:
      each weight moves by <= U_BF16 relative, so column c moves by
      <= U_BF16 * A[c], A[c] = sum_t w_t |V_t[c]| (w = the softmax weights);
    * the fp32 scores carry <= 576 * U_F32 * softmax_scale * sum_d |q_d k_d|
      (any order of the 576-term sum) plus fp32 rounding of the scaled
      score, the exp2 and the base-2 references (<= 2^-16 in all, in natural-log
      units): Delta.  Weights then move by <= e^(2 Delta) - 1 ~ 2 Delta
      relative, i.e. <= 2 Delta * A[c] on column c;
    * the output is rounded to bf16 once: <= U_BF16 * |out|.

    Returns float64 [R, 512]: U_BF16 |ref| + (1 + U_BF16)(U_BF16 + 2.01 Delta) A + 1e-7."""
    R = qrows.shape[0]
    if keys.shape[0] == 0:
        return np.full((R, 512), 1e-7)
    S = (qrows @ keys.T) * scale
    m = S.max(axis=1, keepdims=True)
    w = np.exp(S - m)
    w /= w.sum(axis=1, keepdims=True)
    vabs = np.abs(keys[:, :512])
    A = w @ vabs
    ref = np.abs(w @ keys[:, :512])
    mag = (np.abs(qrows) @ np.abs(keys).T).max(axis=1, keepdims=True)
    delta = scale * 576 * U_F32 * mag + np.abs(S).max(axis=1, keepdims=True) * 2 * U_F32 + 2.0 ** -16
    return U_BF16 * ref + (1 + U_BF16) * (U_BF16 + 2.01 * delta) * A + 1e-7


def dense_out_bound(inp, causal=False, kv=None):
    """row_out_bound for every (request, query token, head) of a dense decode,
    as float64 [b, s_q, h_q, 512]; ``kv`` replaces inp.kv_cache (the
    dequantized cache of an FP8 test)."""
    import oracle
    kv = inp.kv_cache if kv is None else kv
    b, s_q, h_q = inp.batch, inp.s_q, inp.h_q
    tol = np.empty((b, s_q, h_q, 512))
    for i in range(b):
        L = int(inp.cache_seqlens[i])
        keys = oracle.request_keys(kv, inp.block_table[i], L)
        for s in range(s_q):
            n = L if not causal else max(0, L - (s_q - 1 - s))
            tol[i, s] = row_out_bound(oracle.bf16_to_f64(inp.q[i, s]), keys[:n], inp.softmax_scale)
    return tol


def sparse_out_bound(inp, indices=None, topk_length="inp", kv=None):
    """row_out_bound for every (request, query token, head) of a sparse decode."""
    import oracle
    idx = inp.indices if indices is None else indices
    tl = inp.topk_length if isinstance(topk_length, str) else topk_length
    kv = inp.kv_cache if kv is None else kv
    b, s_q, topk = idx.shape
    tol = np.empty((b, s_q, inp.q.shape[2], 512))
    for i in range(b):
        n = topk if tl is None else min(max(int(tl[i]), 0), topk)
        for s in range(s_q):
            keys = oracle.sparse_keys(kv, idx[i, s], n)
            tol[i, s] = row_out_bound(oracle.bf16_to_f64(inp.q[i, s]), keys, inp.softmax_scale)
    return tol


def max_err(a, b):
    """Max |a - b|, treating matching infinities as equal."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    same_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    with np.errstate(invalid="ignore"):
        d = np.where(same_inf, 0.0, np.abs(a - b))
    d = np.where(np.isnan(d), np.inf, d)
    return float(d.max()) if d.size else 0.0


def assert_parity(out, lse, ref_out, ref_lse, what="", out_tol=OUT_TOL):
    """max |out - ref| within out_tol (a number, or an elementwise bound of
    out's shape) and max |lse - ref| within LSE_TOL; prints the errors and the
    margins (tolerance minus error; for an elementwise bound, the smallest)."""
    tol = np.broadcast_to(np.asarray(out_tol, np.float64), np.shape(out))
    a = np.asarray(out, np.float64)
    b = np.asarray(ref_out, np.float64)
    same_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    with np.errstate(invalid="ignore"):
        d = np.where(same_inf, 0.0, np.abs(a - b))
    d = np.where(np.isnan(d), np.inf, d)
    eo = float(d.max()) if d.size else 0.0
    out_margin = float((tol - d).min()) if d.size else 0.0
    worst = float((d / tol).max()) if d.size else 0.0
    el = max_err(lse, ref_lse)
    finite = np.isfinite(b)
    rms = float(np.sqrt(np.mean((a[finite] - b[finite]) ** 2)) /
                max(1e-30, np.sqrt(np.mean(b[finite] ** 2)))) if finite.any() else 0.0
    kind = f"{float(out_tol):.1e}" if np.ndim(out_tol) == 0 else f"elementwise bound, max {float(tol.max()):.2e}"
    print(f"[parity] {what}: max|dout|={eo:.3e} (tol {kind}; margin {out_margin:.3e}, worst err/tol {worst:.3f}) "
          f"max|dlse|={el:.3e} (tol {LSE_TOL:.0e}; margin {LSE_TOL - el:.3e}) rms_rel_out={rms:.3e}", flush=True)
    assert out_margin >= 0, f"{what}: |out - ref| exceeds its bound (worst err/tol {worst}, max err {eo})"
    assert el <= LSE_TOL, f"{what}: max|lse - ref| = {el}"
