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


from oracle.tolerance import U_BF16, U_F32, dense_out_bound, row_out_bound, sparse_out_bound  # noqa: F401,E402


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
