"""Host-side tests of the C-ABI library (no GPU needed): it loads, exports
every symbol include/*.h declares, its planner agrees bit for bit with the
reference planner, and argument errors come back as error codes."""
import ctypes
import glob
import os
import re

import numpy as np
import pytest

import decode_attention_mla_amd as mla
import oracle
from decode_attention_mla_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = []
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(mla_[a-z_]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_library_loads_and_exports_every_declared_symbol():
    L = mla.lib()
    decl = declared_functions()
    assert set(decl) == set(binding.EXPORTED), decl
    for name in decl:
        assert hasattr(L, name), f"{name} not exported"
        ctypes.cast(getattr(L, name), ctypes.c_void_p)


@pytest.mark.parametrize("seed", range(30))
def test_planner_bit_exact_with_reference(seed):
    rng = np.random.default_rng(100 + seed)
    b = int(rng.integers(1, 160))
    kind = seed % 3
    if kind == 0:
        sl = rng.integers(0, 20000, size=b)
    elif kind == 1:
        sl = rng.integers(512, 16385, size=b)
    else:
        sl = np.where(rng.random(b) < 0.2, rng.integers(60000, 140000, size=b), rng.integers(1, 900, size=b))
    P = int(rng.integers(1, 400))
    F = int(rng.integers(0, 8))
    s_ref, n_ref = oracle.plan(sl, num_parts=P, fixed_overhead=F)
    s_lib, n_lib = mla.mla_plan(sl, num_parts=P, fixed_overhead=F)
    assert np.array_equal(s_ref, s_lib) and np.array_equal(n_ref, n_lib)
    k = int(rng.integers(1, 6))
    s_ref, n_ref = oracle.plan(sl, num_parts=P, force_splits=k)
    s_lib, n_lib = mla.mla_plan(sl, num_parts=P, force_splits=k)
    assert np.array_equal(s_ref, s_lib) and np.array_equal(n_ref, n_lib)


@pytest.mark.parametrize("h_q,s_q", [(16, 1), (128, 1), (128, 2), (64, 1), (8, 3)])
def test_get_metadata_policy_matches_reference_plan(h_q, s_q):
    sl = np.array([100, 257, 4096, 0, 70000, 1], dtype=np.int32)
    sched, ns, total = mla.get_mla_metadata_host(sl, h_q, s_q, num_cus=256)
    R = h_q * s_q
    groups = 1 if R <= 16 else -(-R // 128) if R >= 128 else -(-R // 32)
    parts = max(1, 256 // groups)
    F = 3 if R <= 16 else 4 if R >= 128 else 2
    s_ref, n_ref = oracle.plan(sl, num_parts=parts, fixed_overhead=F)
    assert np.array_equal(sched, s_ref) and np.array_equal(ns, n_ref) and total == n_ref[-1]
    assert total <= sched.shape[0] + len(sl) - 1


def test_workspace_bytes():
    # 3 slots x 128 rows = 384 partial rows: 384 x 512 fp32 = 786432 B
    # (256-aligned) plus 384 fp32 lse = 1536 B (256-aligned).
    assert mla.mla_workspace_bytes(3, 128, 1) == 786432 + 1536
    assert mla.mla_workspace_bytes(0, 128, 1) == 0
    # 2 slots x 24 rows = 48 rows: 48 x 2048 = 98304 B, 48 x 4 = 192 -> 256.
    assert mla.mla_workspace_bytes(2, 12, 2) == 98304 + 256


def test_plan_errors():
    with pytest.raises(mla.MlaError, match="< 0"):
        mla.mla_plan([10, -1], num_parts=4)
    with pytest.raises(mla.MlaError):
        mla.mla_plan([10], num_parts=0)
    L = mla.lib()
    sl = np.array([6400, 6400], dtype=np.int32)
    sched = np.zeros((1, 8), dtype=np.int32)
    ns = np.zeros(3, dtype=np.int32)
    n = ctypes.c_int(0)
    p32 = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))  # noqa: E731
    rc = L.mla_plan(p32(sl), 2, 4, 0, 0, p32(sched), 1, p32(ns), ctypes.byref(n))
    assert rc == -2 and b"max_parts" in L.mla_last_error()


def test_decode_argument_errors_return_codes_without_launching():
    L = mla.lib()
    rc = L.mla_decode_fwd(None, None, None, None, 1, 1, 16, 1, 1, 0.1, 0, 0, None, 1, None, None, 0, None, None, None)
    assert rc == -1 and b"null" in L.mla_last_error()
    dummy = ctypes.c_void_p(16)   # never dereferenced: every check fails before any launch
    rc = L.mla_decode_fwd(dummy, dummy, dummy, dummy, 0, 1, 16, 1, 1, 0.1, 0, 0, dummy, 1, dummy, dummy, 0,
                          dummy, dummy, None)
    assert rc == -1 and b"batch=0" in L.mla_last_error()
    rc = L.mla_decode_fwd(dummy, dummy, dummy, dummy, 2, 1, 16, 8, 4, float("nan"), 0, 0, dummy, 3, dummy, dummy, 0,
                          dummy, dummy, None)
    assert rc == -1 and b"softmax_scale" in L.mla_last_error()
    rc = L.mla_decode_fwd(dummy, dummy, dummy, dummy, 2, 1, 16, 8, 4, 0.1, 2, 0, dummy, 3, dummy, dummy, 0,
                          dummy, dummy, None)
    assert rc == -1 and b"causal" in L.mla_last_error()
    rc = L.mla_decode_fwd(dummy, dummy, dummy, dummy, 2, 1, 16, 8, 4, 0.1, 0, 0, dummy, 3, dummy, dummy, 100,
                          dummy, dummy, None)
    assert rc == -3 and b"workspace" in L.mla_last_error()
    rc = L.mla_decode_fwd(dummy, dummy, dummy, dummy, 2, 1, 16, 8, 4, 0.1, 0, 2, dummy, 3, dummy, dummy, 0,
                          dummy, dummy, None)
    assert rc == -1 and b"is_fp8" in L.mla_last_error()


def test_device_planner_argument_errors_return_codes_without_launching():
    L = mla.lib()
    dummy = ctypes.c_void_p(16)   # never dereferenced: every check fails before any launch
    n = ctypes.c_int(0)
    rc = L.mla_get_metadata_device(dummy, 4, 16, 1, 256, None, 256, dummy, ctypes.byref(n), None)
    assert rc == -1 and b"null" in L.mla_last_error()
    rc = L.mla_get_metadata_device(dummy, 70000, 16, 1, 256, dummy, 256, dummy, ctypes.byref(n), None)
    assert rc == -1 and b"batch" in L.mla_last_error()
    rc = L.mla_get_metadata_device(dummy, 4, 16, 1, 256, dummy, 255, dummy, ctypes.byref(n), None)
    assert rc == -2 and b"max_parts" in L.mla_last_error()
    rc = L.mla_get_metadata_device(dummy, 4, 16, 1, 5000, dummy, 5000, dummy, ctypes.byref(n), None)
    assert rc == -1 and b"4096" in L.mla_last_error()


@pytest.mark.parametrize("h_q,s_q,topk_length", [(16, 1, None), (16, 2, [100, 0, 5000, 64]), (64, 2, None),
                                                 (128, 2, [3000, 1, -5, 4096]), (256, 1, [64, 65, 129, 2048])])
def test_sparse_policy_matches_reference_plan_over_token_lists(h_q, s_q, topk_length):
    """The sparse plan walks one request per (request, query token), of length
    the entries that count, with the 128-row kernel's policy above 16 rows."""
    b, topk = 4, 4096
    sched, ns, total = mla.get_mla_metadata_sparse_host(topk_length, b, s_q, h_q, topk, num_cus=256)
    lens = []
    for i in range(b):
        n = topk if topk_length is None else min(max(topk_length[i], 0), topk)
        lens += [n] * s_q
    groups = 1 if h_q <= 16 else -(-h_q // 128)
    F = 3 if h_q <= 16 else 4
    s_ref, n_ref = oracle.plan(np.array(lens, dtype=np.int32), num_parts=max(1, 256 // groups), fixed_overhead=F)
    assert np.array_equal(sched, s_ref) and np.array_equal(ns, n_ref) and total == n_ref[-1]


def test_sparse_argument_errors_return_codes_without_launching():
    L = mla.lib()
    dummy = ctypes.c_void_p(16)   # never dereferenced: every check fails before any launch
    rc = L.mla_decode_sparse_fwd(None, dummy, dummy, None, 1, 1, 16, 1, 64, 0.1, 0, dummy, 1, dummy, dummy, 1 << 30,
                                 dummy, dummy, None)
    assert rc == -1 and b"null" in L.mla_last_error()
    rc = L.mla_decode_sparse_fwd(dummy, dummy, dummy, None, 1, 1, 16, 1, 0, 0.1, 0, dummy, 1, dummy, dummy, 1 << 30,
                                 dummy, dummy, None)
    assert rc == -1 and b"topk=0" in L.mla_last_error()
    rc = L.mla_decode_sparse_fwd(dummy, dummy, dummy, None, 1, 1, 16, (1 << 24) + 1, 64, 0.1, 0, dummy, 1, dummy, dummy,
                                 1 << 30, dummy, dummy, None)
    assert rc == -1 and b"num_blocks" in L.mla_last_error()
    rc = L.mla_decode_sparse_fwd(dummy, dummy, dummy, None, 2, 2, 16, 8, 64, -1.0, 0, dummy, 3, dummy, dummy, 1 << 30,
                                 dummy, dummy, None)
    assert rc == -1 and b"softmax_scale" in L.mla_last_error()
    rc = L.mla_decode_sparse_fwd(dummy, dummy, dummy, None, 2, 2, 16, 8, 64, 0.1, 0, dummy, 3, dummy, dummy, 100,
                                 dummy, dummy, None)
    assert rc == -3 and b"workspace" in L.mla_last_error()
    rc = L.mla_decode_sparse_fwd(dummy, dummy, dummy, None, 2, 2, 16, 8, 64, 0.1, 3, dummy, 3, dummy, dummy, 1 << 30,
                                 dummy, dummy, None)
    assert rc == -1 and b"is_fp8" in L.mla_last_error()
    with pytest.raises(mla.MlaError, match="topk"):
        mla.get_mla_metadata_sparse_host(None, 2, 1, 16, 0, num_cus=8)


def test_entry_points_raise_without_the_library():
    """No CPU fallback: with the library missing, every entry point raises
    (checked in a fresh interpreter, so the loaded library does not leak)."""
    import subprocess
    import sys
    code = (
        "import numpy as np\n"
        "from decode_attention_mla_amd import binding\n"
        "binding.LIB_PATH = '/nonexistent/libmla_decode.so'\n"
        "calls = [lambda: binding.get_mla_metadata_host(np.array([100], np.int32), 16, 1),\n"
        "         lambda: binding.mla_plan(np.array([100], np.int32), 4),\n"
        "         lambda: binding.mla_workspace_bytes(4, 16, 1),\n"
        "         lambda: binding.get_mla_metadata_sparse_host(None, 1, 1, 16, 64)]\n"
        "for c in calls:\n"
        "    try:\n"
        "        c()\n"
        "    except RuntimeError as e:\n"
        "        assert 'missing' in str(e), e\n"
        "    else:\n"
        "        raise SystemExit('an entry point ran without the library')\n"
        "print('raised')\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    res = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=120)
    assert res.returncode == 0 and "raised" in res.stdout, res.stdout + res.stderr
