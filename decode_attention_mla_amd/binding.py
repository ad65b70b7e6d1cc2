"""Thin ctypes binding of ``libmla_decode.so`` (argument marshalling only).

Every step of the decode runs in the HIP library; this module checks Python
arguments, allocates outputs and scratch with PyTorch (device memory and
streams only) and calls the C ABI declared in ``include/mla_decode.h``.
There is no fallback: if the library is missing, every entry point raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmla_decode.so")
SCHED_INTS = 8
PAGE = 64
D_QK = 576
D_V = 512
FP8_RECORD = 656   # bytes per token of an FP8 cache (512 e4m3 + 4 fp32 scales + 64 bf16)

# Every symbol include/mla_decode.h declares.
EXPORTED = ("mla_plan", "mla_get_metadata", "mla_plan_attach_pages", "mla_get_metadata_device", "mla_max_parts",
            "mla_workspace_bytes",
            "mla_decode_fwd", "mla_decode_fwd_noalloc", "mla_max_parts_sparse", "mla_get_metadata_sparse", "mla_decode_sparse_fwd",
            "mla_profile_start", "mla_profile_stop", "mla_last_error")

_lib = None


class MlaError(RuntimeError):
    """A non-zero return code from the library, with its message."""


def lib() -> ctypes.CDLL:
    """Load the library once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                           "or python -m decode_attention_mla_amd.build")
    # PyTorch's ROCm build ships its own HIP runtime: load it first, so that the
    # library binds to the runtime the tensors live in (a library loaded first
    # binds to another copy, whose device queries then fail once torch loads).
    import torch  # noqa: F401
    L = ctypes.CDLL(LIB_PATH)
    i32p = ctypes.POINTER(ctypes.c_int32)
    ip = ctypes.POINTER(ctypes.c_int)
    vp = ctypes.c_void_p
    L.mla_plan.argtypes = [i32p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, i32p,
                           ctypes.c_int, i32p, ip]
    L.mla_plan.restype = ctypes.c_int
    L.mla_get_metadata.argtypes = [i32p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, i32p, ctypes.c_int, i32p, ip, ip]
    L.mla_get_metadata.restype = ctypes.c_int
    L.mla_max_parts.argtypes = [i32p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                ctypes.c_int]
    L.mla_max_parts.restype = ctypes.c_int
    L.mla_workspace_bytes.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    L.mla_workspace_bytes.restype = ctypes.c_size_t
    L.mla_plan_attach_pages.argtypes = [i32p, ctypes.c_int, i32p, ctypes.c_int, i32p, ctypes.c_int, ctypes.c_int]
    L.mla_plan_attach_pages.restype = ctypes.c_int
    L.mla_get_metadata_device.argtypes = [vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          vp, ctypes.c_int, vp, vp, ctypes.c_int, ctypes.c_int, ip, vp]
    L.mla_get_metadata_device.restype = ctypes.c_int
    L.mla_decode_fwd.argtypes = [vp, vp, vp, vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_int, ctypes.c_float, ctypes.c_int, ctypes.c_int, vp, ctypes.c_int, vp, vp,
                                 ctypes.c_size_t, vp, vp, vp]
    L.mla_decode_fwd.restype = ctypes.c_int
    L.mla_decode_fwd_noalloc.argtypes = [vp, vp, vp, vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_float, ctypes.c_int, ctypes.c_int, vp, ctypes.c_int, vp,
                                         vp, vp, vp]
    L.mla_decode_fwd_noalloc.restype = ctypes.c_int
    L.mla_max_parts_sparse.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int]
    L.mla_max_parts_sparse.restype = ctypes.c_int
    L.mla_get_metadata_sparse.argtypes = [i32p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          i32p, ctypes.c_int, i32p, ip, ip]
    L.mla_get_metadata_sparse.restype = ctypes.c_int
    L.mla_decode_sparse_fwd.argtypes = [vp, vp, vp, vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_float, ctypes.c_int, vp, ctypes.c_int, vp, vp,
                                        ctypes.c_size_t, vp, vp, vp]
    L.mla_decode_sparse_fwd.restype = ctypes.c_int
    L.mla_profile_start.argtypes = [ctypes.c_int]
    L.mla_profile_start.restype = ctypes.c_int
    fp = ctypes.POINTER(ctypes.c_float)
    L.mla_profile_stop.argtypes = [fp, fp, ip]
    L.mla_profile_stop.restype = ctypes.c_int
    L.mla_last_error.argtypes = []
    L.mla_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(rc: int, name: str) -> None:
    if rc != 0:
        raise MlaError(f"{name} returned {rc}: {lib().mla_last_error().decode()}")


def _i32_host(x) -> np.ndarray:
    if hasattr(x, "detach"):            # torch tensor (host or device)
        x = x.detach().to("cpu").numpy()
    a = np.ascontiguousarray(np.asarray(x), dtype=np.int32)
    return a


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


# ---------------------------------------------------------------------------
# Planning (host)

def mla_plan(cache_seqlens, num_parts: int, fixed_overhead: int = 0, force_splits: int = 0):
    """Host planner with explicit parts / overhead: (sched int32 [P, 8], num_splits int32 [b + 1])."""
    sl = _i32_host(cache_seqlens)
    b = int(sl.shape[0])
    cap = max(1, num_parts) if force_splits <= 0 else int(sum(max(1, min(force_splits, (int(L) + PAGE - 1) // PAGE)) for L in sl))
    sched = np.zeros((cap, SCHED_INTS), dtype=np.int32)
    ns = np.zeros(b + 1, dtype=np.int32)
    nparts = ctypes.c_int(0)
    _check(lib().mla_plan(_ptr(sl), b, int(num_parts), int(fixed_overhead), int(force_splits), _ptr(sched), cap,
                          _ptr(ns), ctypes.byref(nparts)), "mla_plan")
    return sched[:nparts.value].copy(), ns


def get_mla_metadata_host(cache_seqlens, h_q: int, s_q: int, num_cus: int = 0, force_splits: int = 0,
                          fp8: bool = False, block_table=None, num_blocks: int = 0):
    """mla_get_metadata on host arrays: (sched [P, 8], num_splits [b + 1], total_splits).
    ``fp8``: the plan serves decode calls on an FP8 cache.  With ``block_table``
    (int32 [b, max_blocks], the decode calls' table; host array or tensor) and
    ``num_blocks`` (the pool's block count) each part's first page is attached
    (mla_plan_attach_pages)."""
    sl = _i32_host(cache_seqlens)
    b = int(sl.shape[0])
    L = lib()
    f8 = 1 if fp8 else 0
    cap = L.mla_max_parts(_ptr(sl), b, int(h_q), int(s_q), f8, int(num_cus), int(force_splits))
    _check(cap if cap < 0 else 0, "mla_max_parts")
    sched = np.zeros((max(cap, 1), SCHED_INTS), dtype=np.int32)
    ns = np.zeros(b + 1, dtype=np.int32)
    nparts = ctypes.c_int(0)
    total = ctypes.c_int(0)
    _check(L.mla_get_metadata(_ptr(sl), b, int(h_q), int(s_q), f8, int(num_cus), int(force_splits), _ptr(sched),
                              sched.shape[0], _ptr(ns), ctypes.byref(nparts), ctypes.byref(total)),
           "mla_get_metadata")
    sched = sched[:nparts.value].copy()
    if block_table is not None:
        attach_pages(sched, sl, block_table, num_blocks)
    return sched, ns, int(total.value)


def attach_pages(sched: np.ndarray, cache_seqlens, block_table, num_blocks: int) -> np.ndarray:
    """mla_plan_attach_pages on a host plan (int32 [P, 8], modified in place)."""
    _need(isinstance(sched, np.ndarray) and sched.dtype == np.int32 and sched.ndim == 2
          and sched.shape[1] == SCHED_INTS and sched.flags.c_contiguous, "sched must be a contiguous int32 [P, 8] array")
    sl = _i32_host(cache_seqlens)
    bt = np.ascontiguousarray(_i32_host(block_table))
    _need(bt.ndim == 2 and bt.shape[0] == sl.shape[0], "block_table must be int32 [b, max_blocks]")
    _check(lib().mla_plan_attach_pages(_ptr(sched), int(sched.shape[0]), _ptr(sl), int(sl.shape[0]), _ptr(bt),
                                       int(bt.shape[1]), int(num_blocks)), "mla_plan_attach_pages")
    return sched


def get_mla_metadata(cache_seqlens, h_q: int, s_q: int, num_cus: int = 0, force_splits: int = 0,
                     device=None, fp8: bool = False, block_table=None, num_blocks: int = 0):
    """Plan one decode step; returns (sched, num_splits) as int32 device tensors.

    The plan is reusable for every call with the same batch, s_q, h_q, cache
    format (``fp8``) and cache_seqlens (e.g. every layer of one decode step).
    ``cache_seqlens`` may be a host array or a tensor; the planner reads it on
    the host.  Passing the decode calls' ``block_table`` and the pool's
    ``num_blocks`` attaches each part's first page (the plan then also needs
    that table unchanged at those positions).
    """
    import torch
    sched, ns, _ = get_mla_metadata_host(cache_seqlens, h_q, s_q, num_cus, force_splits, fp8, block_table,
                                         num_blocks)
    dev = device if device is not None else torch.device("cuda", torch.cuda.current_device())
    return (torch.from_numpy(sched).to(dev, non_blocking=False),
            torch.from_numpy(ns).to(dev, non_blocking=False))


def get_mla_metadata_device(cache_seqlens, h_q: int, s_q: int, num_cus: int = 0, fp8: bool = False,
                            block_table=None, num_blocks: int = 0):
    """The split plan computed on the GPU from device lengths (int32 [b]),
    enqueued on the current stream: returns (sched int32 [P, 8],
    num_splits int32 [b + 1]) device tensors, P = the policy's part count
    (rows past the walk's last part are empty).  Capturable in a graph.
    With ``block_table`` (int32 [b, max_blocks] GPU tensor) and
    ``num_blocks`` the plan carries each part's first page."""
    import torch
    _need(cache_seqlens.dim() == 1 and cache_seqlens.dtype == torch.int32 and cache_seqlens.is_cuda
          and cache_seqlens.is_contiguous(), "cache_seqlens must be a contiguous int32 [b] GPU tensor")
    bt_ptr, max_blocks = None, 0
    if block_table is not None:
        _need(block_table.dim() == 2 and block_table.dtype == torch.int32 and block_table.is_cuda
              and block_table.is_contiguous() and block_table.shape[0] == cache_seqlens.shape[0],
              "block_table must be a contiguous int32 [b, max_blocks] GPU tensor")
        bt_ptr, max_blocks = block_table.data_ptr(), int(block_table.shape[1])
    b = int(cache_seqlens.shape[0])
    dummy = np.zeros(b, dtype=np.int32)   # the part count depends on sizes only
    f8 = 1 if fp8 else 0
    cap = lib().mla_max_parts(_ptr(dummy), b, int(h_q), int(s_q), f8, int(num_cus), 0)
    _check(cap if cap < 0 else 0, "mla_max_parts")
    dev = cache_seqlens.device
    sched = torch.empty((cap, SCHED_INTS), dtype=torch.int32, device=dev)
    ns = torch.empty(b + 1, dtype=torch.int32, device=dev)
    parts = ctypes.c_int(0)
    stream = torch.cuda.current_stream(dev).cuda_stream
    _check(lib().mla_get_metadata_device(cache_seqlens.data_ptr(), b, int(h_q), int(s_q), f8, int(num_cus),
                                         sched.data_ptr(), cap, ns.data_ptr(), bt_ptr, max_blocks, int(num_blocks),
                                         ctypes.byref(parts), stream),
           "mla_get_metadata_device")
    return sched[:parts.value], ns


def mla_workspace_bytes(total_splits: int, h_q: int, s_q: int) -> int:
    return int(lib().mla_workspace_bytes(int(total_splits), int(h_q), int(s_q)))


# ---------------------------------------------------------------------------
# Decode

def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _kv_check(kv_cache, fp8: bool):
    import torch
    if fp8:
        _need(kv_cache.dim() == 4 and tuple(kv_cache.shape[1:]) == (PAGE, 1, FP8_RECORD) and
              kv_cache.dtype == torch.uint8, f"an FP8 kv_cache must be uint8 [num_blocks, 64, 1, 656], got "
              f"{kv_cache.dtype} {tuple(kv_cache.shape)}")
    else:
        _need(kv_cache.dim() == 4 and tuple(kv_cache.shape[1:]) == (PAGE, 1, D_QK) and
              kv_cache.dtype == torch.bfloat16,
              f"kv_cache must be bf16 [num_blocks, 64, 1, 576], got {kv_cache.dtype} {tuple(kv_cache.shape)}")


def _dense_checks(q, kv_cache, block_table, cache_seqlens, sched, num_splits, out, lse, fp8):
    """Validates a dense decode call; returns (b, s_q, h_q, out, lse), allocating
    out / lse when they are None."""
    import torch
    _need(q.dim() == 4 and q.shape[3] == D_QK, f"q must be [b, s_q, h_q, 576], got {tuple(q.shape)}")
    b, s_q, h_q = (int(x) for x in q.shape[:3])
    _kv_check(kv_cache, fp8)
    _need(block_table.dim() == 2 and block_table.shape[0] == b, "block_table must be [b, max_blocks]")
    _need(cache_seqlens.dim() == 1 and cache_seqlens.shape[0] == b, "cache_seqlens must be [b]")
    _need(sched.dim() == 2 and sched.shape[1] == SCHED_INTS and sched.shape[0] > 0, "sched must be [P, 8]")
    _need(num_splits.dim() == 1 and num_splits.shape[0] == b + 1, "num_splits must be [b + 1]")
    for name, t, dt in (("q", q, torch.bfloat16), ("kv_cache", kv_cache, kv_cache.dtype),
                        ("block_table", block_table, torch.int32), ("cache_seqlens", cache_seqlens, torch.int32),
                        ("sched", sched, torch.int32), ("num_splits", num_splits, torch.int32)):
        _need(t.dtype == dt, f"{name} must be {dt}, got {t.dtype}")
        _need(t.is_cuda and t.device == q.device, f"{name} must be on {q.device}")
        _need(t.is_contiguous(), f"{name} must be contiguous")
    if out is None:
        out = torch.empty((b, s_q, h_q, D_V), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((b, h_q, s_q), dtype=torch.float32, device=q.device)
    _need(out.dtype == torch.bfloat16 and tuple(out.shape) == (b, s_q, h_q, D_V) and out.is_contiguous(),
          "out must be contiguous bf16 [b, s_q, h_q, 512]")
    _need(lse.dtype == torch.float32 and tuple(lse.shape) == (b, h_q, s_q) and lse.is_contiguous(),
          "lse must be contiguous fp32 [b, h_q, s_q]")
    _need(out.device == q.device and lse.device == q.device, f"out and lse must be on {q.device}")
    return b, s_q, h_q, out, lse


def mla_decode_fwd(q, kv_cache, block_table, cache_seqlens, softmax_scale: float, sched, num_splits,
                   out=None, lse=None, workspace=None, causal: bool = False, fp8: bool = False):
    """Dense MLA decode.  Returns (out bf16 [b, s_q, h_q, 512], lse fp32 [b, h_q, s_q]).

    q bf16 [b, s_q, h_q, 576]; kv_cache bf16 [num_blocks, 64, 1, 576], or with
    fp8=True the FP8 records uint8 [num_blocks, 64, 1, 656];
    block_table int32 [b, max_blocks]; cache_seqlens int32 [b];
    sched / num_splits from get_mla_metadata for the same cache_seqlens.
    causal: query token s of s_q sees keys 0 .. L - s_q + s (multi-token
    prediction) instead of all L.
    All tensors on the same GPU, contiguous.  Enqueued on the current stream.
    """
    import torch
    b, s_q, h_q, out, lse = _dense_checks(q, kv_cache, block_table, cache_seqlens, sched, num_splits, out, lse, fp8)
    num_parts = int(sched.shape[0])
    ws_bytes = mla_workspace_bytes(num_parts + b - 1, h_q, s_q)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=q.device)
    _need(workspace.numel() * workspace.element_size() >= ws_bytes, f"workspace needs {ws_bytes} bytes")
    stream = torch.cuda.current_stream(q.device).cuda_stream
    rc = lib().mla_decode_fwd(q.data_ptr(), kv_cache.data_ptr(), block_table.data_ptr(), cache_seqlens.data_ptr(),
                              b, s_q, h_q, int(kv_cache.shape[0]), int(block_table.shape[1]),
                              float(softmax_scale), 1 if causal else 0, 1 if fp8 else 0, sched.data_ptr(), num_parts,
                              num_splits.data_ptr(),
                              workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                              out.data_ptr(), lse.data_ptr(), stream)
    _check(rc, "mla_decode_fwd")
    return out, lse


def mla_decode_fwd_noalloc(q, kv_cache, block_table, cache_seqlens, softmax_scale: float, sched, num_splits, out, lse,
                           causal: bool = False, fp8: bool = False):
    """mla_decode_fwd without a workspace argument: the library's own
    per-GPU split array serves (``mla_decode_fwd_noalloc``; plans needing more
    than MLA_NOALLOC_SCRATCH_BYTES are rejected).  ``out`` and ``lse`` are
    caller buffers (nothing is allocated here either).  Calls that overlap
    on one GPU race on that array."""
    import torch
    _need(out is not None and lse is not None, "mla_decode_fwd_noalloc writes into caller buffers: pass out and lse")
    b, s_q, h_q, out, lse = _dense_checks(q, kv_cache, block_table, cache_seqlens, sched, num_splits, out, lse, fp8)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    rc = lib().mla_decode_fwd_noalloc(q.data_ptr(), kv_cache.data_ptr(), block_table.data_ptr(),
                                      cache_seqlens.data_ptr(), b, s_q, h_q, int(kv_cache.shape[0]),
                                      int(block_table.shape[1]), float(softmax_scale), 1 if causal else 0,
                                      1 if fp8 else 0, sched.data_ptr(), int(sched.shape[0]), num_splits.data_ptr(),
                                      out.data_ptr(), lse.data_ptr(), stream)
    _check(rc, "mla_decode_fwd_noalloc")
    return out, lse


# ---------------------------------------------------------------------------
# Sparse (top-k) decode

def get_mla_metadata_sparse_host(topk_length, batch: int, s_q: int, h_q: int, topk: int, num_cus: int = 0):
    """mla_get_metadata_sparse: (sched [P, 8], num_splits [b * s_q + 1],
    total_splits) host arrays.  topk_length: host int32 [b] or None."""
    L = lib()
    cap = L.mla_max_parts_sparse(int(batch), int(s_q), int(h_q), int(num_cus))
    _check(cap if cap < 0 else 0, "mla_max_parts_sparse")
    sched = np.zeros((max(cap, 1), SCHED_INTS), dtype=np.int32)
    ns = np.zeros(int(batch) * int(s_q) + 1, dtype=np.int32)
    nparts, total = ctypes.c_int(0), ctypes.c_int(0)
    tl = None if topk_length is None else _i32_host(topk_length)
    _check(L.mla_get_metadata_sparse(None if tl is None else _ptr(tl), int(batch), int(s_q), int(h_q), int(topk),
                                     int(num_cus), _ptr(sched), sched.shape[0], _ptr(ns), ctypes.byref(nparts),
                                     ctypes.byref(total)), "mla_get_metadata_sparse")
    return sched[:nparts.value].copy(), ns, int(total.value)


def get_mla_metadata_sparse(topk_length, batch: int, s_q: int, h_q: int, topk: int, device=None, num_cus: int = 0):
    """The sparse plan as device tensors (sched int32 [P, 8], num_splits int32 [b * s_q + 1])."""
    import torch
    sched, ns, _ = get_mla_metadata_sparse_host(topk_length, batch, s_q, h_q, topk, num_cus)
    dev = device if device is not None else torch.device("cuda", torch.cuda.current_device())
    return torch.from_numpy(sched).to(dev), torch.from_numpy(ns).to(dev)


def mla_decode_sparse_fwd(q, kv_cache, indices, softmax_scale: float, sched, num_splits, topk_length=None,
                          out=None, lse=None, workspace=None, fp8: bool = False):
    """Sparse MLA decode.  Returns (out bf16 [b, s_q, h_q, 512], lse fp32 [b, h_q, s_q]).

    q bf16 [b, s_q, h_q, 576]; kv_cache bf16 [num_blocks, 64, 1, 576];
    indices int32 [b, s_q, topk] (page_id * 64 + offset; out-of-range
    entries name no key); topk_length int32 [b] (device) or None;
    sched / num_splits from get_mla_metadata_sparse with the same sizes and
    topk_length.  All tensors on the same GPU, contiguous; enqueued on the
    current stream.
    """
    import torch
    _need(q.dim() == 4 and q.shape[3] == D_QK, f"q must be [b, s_q, h_q, 576], got {tuple(q.shape)}")
    b, s_q, h_q = (int(x) for x in q.shape[:3])
    _kv_check(kv_cache, fp8)
    _need(indices.dim() == 3 and tuple(indices.shape[:2]) == (b, s_q) and indices.shape[2] > 0,
          "indices must be [b, s_q, topk]")
    topk = int(indices.shape[2])
    n = b * s_q
    _need(sched.dim() == 2 and sched.shape[1] == SCHED_INTS and sched.shape[0] > 0, "sched must be [P, 8]")
    _need(num_splits.dim() == 1 and num_splits.shape[0] == n + 1, "num_splits must be [b * s_q + 1]")
    checks = [("q", q, torch.bfloat16), ("kv_cache", kv_cache, kv_cache.dtype), ("indices", indices, torch.int32),
              ("sched", sched, torch.int32), ("num_splits", num_splits, torch.int32)]
    if topk_length is not None:
        _need(topk_length.dim() == 1 and topk_length.shape[0] == b, "topk_length must be [b]")
        checks.append(("topk_length", topk_length, torch.int32))
    for name, t, dt in checks:
        _need(t.dtype == dt, f"{name} must be {dt}, got {t.dtype}")
        _need(t.is_cuda and t.device == q.device, f"{name} must be on {q.device}")
        _need(t.is_contiguous(), f"{name} must be contiguous")
    num_parts = int(sched.shape[0])
    if out is None:
        out = torch.empty((b, s_q, h_q, D_V), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((b, h_q, s_q), dtype=torch.float32, device=q.device)
    _need(out.dtype == torch.bfloat16 and tuple(out.shape) == (b, s_q, h_q, D_V) and out.is_contiguous(),
          "out must be contiguous bf16 [b, s_q, h_q, 512]")
    _need(lse.dtype == torch.float32 and tuple(lse.shape) == (b, h_q, s_q) and lse.is_contiguous(),
          "lse must be contiguous fp32 [b, h_q, s_q]")
    ws_bytes = mla_workspace_bytes(num_parts + n - 1, h_q, 1)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=q.device)
    _need(workspace.numel() * workspace.element_size() >= ws_bytes, f"workspace needs {ws_bytes} bytes")
    stream = torch.cuda.current_stream(q.device).cuda_stream
    rc = lib().mla_decode_sparse_fwd(q.data_ptr(), kv_cache.data_ptr(), indices.data_ptr(),
                                     None if topk_length is None else topk_length.data_ptr(),
                                     b, s_q, h_q, int(kv_cache.shape[0]), topk, float(softmax_scale),
                                     1 if fp8 else 0, sched.data_ptr(), num_parts, num_splits.data_ptr(), workspace.data_ptr(),
                                     workspace.numel() * workspace.element_size(), out.data_ptr(), lse.data_ptr(),
                                     stream)
    _check(rc, "mla_decode_sparse_fwd")
    return out, lse


def profile_start(max_calls: int) -> None:
    """Record per-kernel HIP events for the next max_calls mla_decode_fwd calls."""
    _check(lib().mla_profile_start(int(max_calls)), "mla_profile_start")


def profile_stop():
    """Return (main_ms_total, combine_ms_total, calls) for the recorded calls."""
    a, c, n = ctypes.c_float(0), ctypes.c_float(0), ctypes.c_int(0)
    _check(lib().mla_profile_stop(ctypes.byref(a), ctypes.byref(c), ctypes.byref(n)), "mla_profile_stop")
    return float(a.value), float(c.value), int(n.value)
