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


def out_tol_bound(inp):
    """Output tolerance derived from the arithmetic for inputs outside the five
    workloads: P is rounded to bf16 for the PV product (<= 2^-9 relative per
    weight, normalised by the fp32 row sum) and out is rounded to bf16
    (<= 2^-9 |out|), so |out - ref| <= 2^-8 max|V| + fp32 accumulation error.
    Never looser than the workloads' 1e-2."""
    from decode_attention_mla_amd import workloads as W
    vmax = 0.0
    for b in range(inp.batch):
        L = int(inp.cache_seqlens[b])
        for j in range((L + 63) // 64):
            rows = inp.kv_cache[inp.block_table[b, j], :min(64, L - 64 * j), 0, :512]
            vmax = max(vmax, float(np.abs(W.bf16_bits_to_f32(rows)).max()))
    return max(OUT_TOL, 2.0 ** -8 * vmax + 1e-4)


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
    eo = max_err(out, ref_out)
    el = max_err(lse, ref_lse)
    finite = np.isfinite(ref_out)
    rms = float(np.sqrt(np.mean((out[finite] - ref_out[finite]) ** 2)) /
                max(1e-30, np.sqrt(np.mean(ref_out[finite] ** 2)))) if finite.any() else 0.0
    print(f"[parity] {what}: max|dout|={eo:.3e} (tol {out_tol:.3e}) max|dlse|={el:.3e} rms_rel_out={rms:.3e}",
          flush=True)
    assert eo <= out_tol, f"{what}: max|out - ref| = {eo} > {out_tol}"
    assert el <= LSE_TOL, f"{what}: max|lse - ref| = {el}"
