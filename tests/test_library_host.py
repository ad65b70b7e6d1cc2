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


def declared_functions(header):
    text = open(os.path.join(ROOT, "include", header)).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(mla_[a-z_]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_every_header_is_checked():
    assert sorted(os.path.basename(h) for h in glob.glob(os.path.join(ROOT, "include", "*.h"))) == \
        ["mla_bench.h", "mla_decode.h"]


def test_library_loads_and_exports_every_declared_symbol():
    L = mla.lib()
    decl = declared_functions("mla_decode.h")
    assert set(decl) == set(binding.EXPORTED), decl
    for name in decl:
        assert hasattr(L, name), f"{name} not exported"
        ctypes.cast(getattr(L, name), ctypes.c_void_p)


def test_bench_library_loads_and_exports_every_declared_symbol():
    from decode_attention_mla_amd import build
    B = ctypes.CDLL(build.BENCH_LIB_PATH)
    decl = declared_functions("mla_bench.h")
    assert set(decl) == {"mla_bench_stream_read", "mla_bench_empty", "mla_bench_last_error"}, decl
    for name in decl:
        assert hasattr(B, name), f"{name} not exported"
    B.mla_bench_last_error.restype = ctypes.c_char_p
    B.mla_bench_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                        ctypes.c_void_p]
    assert B.mla_bench_stream_read(None, 1024, None, 4, None) == -1      # rejected before any launch
    assert b"bad argument" in B.mla_bench_last_error()


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


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("h_q,s_q", [(16, 1), (128, 1), (128, 2), (64, 1), (8, 3), (24, 2)])
def test_get_metadata_policy_matches_reference_plan(h_q, s_q, fp8):
    """The policy's part count and overhead by kernel geometry: an FP8 cache
    takes the 128-row kernel above 16 rows, so its plan has one part per CU
    there (every CU gets a workgroup) rather than the 32-row kernel's."""
    sl = np.array([100, 257, 4096, 0, 70000, 1], dtype=np.int32)
    sched, ns, total = mla.get_mla_metadata_host(sl, h_q, s_q, num_cus=256, fp8=fp8)
    R = h_q * s_q
    wide = R >= 128 or (fp8 and R > 16)
    groups = 1 if R <= 16 else -(-R // 128) if wide else -(-R // 32)
    parts = max(1, 256 // groups)
    if fp8 and 16 < R < 128:
        assert parts == 256
    F = 3 if R <= 16 else (6 if groups >= 2 else 4) if wide else 2
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


def _expected_first_pages(sched, seqlens, table):
    """Column 6 written out from the plan row's meaning: the part's first
    piece covers pages begin_block .. (end_block if it ends in the same
    request, else that request's last page) of begin_req."""
    want = np.zeros(sched.shape[0], dtype=np.int32)
    for q, (br, er, bb, eb) in enumerate(sched[:, :4]):
        if br > er:
            continue
        end = eb if br == er else -(-int(seqlens[br]) // 64)
        if bb < end:
            want[q] = table[br, bb] + 1
    return want


@pytest.mark.parametrize("seed", range(12))
def test_attach_pages_writes_each_parts_first_block_id(seed):
    rng = np.random.default_rng(300 + seed)
    b = int(rng.integers(1, 70))
    sl = rng.integers(0, 9000, size=b).astype(np.int32)
    sl[rng.random(b) < 0.25] = 0                               # empty requests: parts with no page
    max_blocks = int(-(-sl.max() // 64)) + int(rng.integers(1, 4))
    num_blocks = b * max_blocks
    table = rng.permutation(num_blocks).astype(np.int32).reshape(b, max_blocks)
    for force in (0, int(rng.integers(1, 6))):
        sched, ns, _ = mla.get_mla_metadata_host(sl, 16, 1, num_cus=int(rng.integers(1, 300)), force_splits=force)
        plain = sched.copy()
        assert np.all(plain[:, 6] == 0)
        mla.binding.attach_pages(sched, sl, table, num_blocks)
        assert np.array_equal(sched[:, [0, 1, 2, 3, 4, 5, 7]], plain[:, [0, 1, 2, 3, 4, 5, 7]])
        want = _expected_first_pages(plain, sl, table)
        assert np.array_equal(sched[:, 6], want)
        nonempty = (plain[:, 0] <= plain[:, 1])
        # every part whose first piece holds pages starts on one (an empty
        # request as the first piece leaves the column 0)
        assert np.all((sched[:, 6] > 0) <= nonempty)
        mla.binding.attach_pages(sched, sl, table, num_blocks)  # idempotent
        assert np.array_equal(sched[:, 6], want)


def test_attach_pages_through_get_metadata_equals_attaching_afterwards():
    sl = np.array([100, 0, 257, 4096, 1], dtype=np.int32)
    table = (np.arange(5 * 64, dtype=np.int32).reshape(5, 64) * 7) % 320
    a, na, ta = mla.get_mla_metadata_host(sl, 16, 1, num_cus=64, block_table=table, num_blocks=320)
    b, nb, tb = mla.get_mla_metadata_host(sl, 16, 1, num_cus=64)
    mla.binding.attach_pages(b, sl, table, 320)
    assert np.array_equal(a, b) and np.array_equal(na, nb) and ta == tb
    assert a[0, 6] == table[0, 0] + 1


def test_attach_pages_errors():
    L = mla.lib()
    p32 = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))  # noqa: E731
    sl = np.array([200, 64], dtype=np.int32)
    sched, _, _ = mla.get_mla_metadata_host(sl, 16, 1, num_cus=2)
    table = np.array([[0, 1, 2, 3], [4, 5, 6, 7]], dtype=np.int32)
    rc = L.mla_plan_attach_pages(None, 2, p32(sl), 2, p32(table), 4, 8)
    assert rc == -1 and b"null" in L.mla_last_error()
    rc = L.mla_plan_attach_pages(p32(sched), sched.shape[0], p32(sl), 2, p32(table), 4, 0)
    assert rc == -1 and b"num_blocks=0" in L.mla_last_error()
    with pytest.raises(mla.MlaError, match="outside"):
        mla.binding.attach_pages(sched.copy(), sl, table, 3)          # id 4 of request 1 is past a 3-block pool
    bad = table.copy()
    bad[0, 0] = -1
    with pytest.raises(mla.MlaError, match="outside"):
        mla.binding.attach_pages(sched.copy(), sl, bad, 8)
    split, _, _ = mla.get_mla_metadata_host(sl, 16, 1, num_cus=2, force_splits=2)
    assert split[1, 0] == 0 and split[1, 2] == 2                      # request 0's second piece starts at page 2
    with pytest.raises(mla.MlaError, match="max_blocks"):
        mla.binding.attach_pages(split, sl, table[:, :2].copy(), 8)
    rows = sched.copy()
    rows[0, 1] = 5                                                    # names request 5 of 2
    with pytest.raises(mla.MlaError, match="names requests"):
        mla.binding.attach_pages(rows, sl, table, 8)


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
    rc = L.mla_get_metadata_device(dummy, 4, 16, 1, 0, 256, None, 256, dummy, None, 0, 0, ctypes.byref(n), None)
    assert rc == -1 and b"null" in L.mla_last_error()
    rc = L.mla_get_metadata_device(dummy, 70000, 16, 1, 0, 256, dummy, 256, dummy, None, 0, 0, ctypes.byref(n), None)
    assert rc == -1 and b"batch" in L.mla_last_error()
    rc = L.mla_get_metadata_device(dummy, 4, 16, 1, 0, 256, dummy, 255, dummy, None, 0, 0, ctypes.byref(n), None)
    assert rc == -2 and b"max_parts" in L.mla_last_error()
    rc = L.mla_get_metadata_device(dummy, 4, 16, 1, 0, 5000, dummy, 5000, dummy, None, 0, 0, ctypes.byref(n), None)
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
    F = 3 if h_q <= 16 else 6 if groups >= 2 else 4
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


def test_lengths_at_the_int32_limit():
    """Lengths up to 2^31 - 1: ceil(L / 64) computed without the int32
    overflow of (L + 63) / 64, by the planner, the part bound and the policy."""
    sl = np.array([2 ** 31 - 1, 100, 2 ** 31 - 64, 2 ** 31 - 65, 0], dtype=np.int32)
    assert [(int(L) + 63) // 64 for L in sl] == [2 ** 25, 2, 2 ** 25 - 1, 2 ** 25 - 1, 0]
    for P, F in ((256, 3), (7, 0), (1, 4)):
        s_ref, n_ref = oracle.plan(sl, num_parts=P, fixed_overhead=F)
        s_lib, n_lib = mla.mla_plan(sl, num_parts=P, fixed_overhead=F)
        assert np.array_equal(s_ref, s_lib) and np.array_equal(n_ref, n_lib)
    s_ref, n_ref = oracle.plan(sl, num_parts=4, force_splits=3)
    s_lib, n_lib = mla.mla_plan(sl, num_parts=4, force_splits=3)
    assert np.array_equal(s_ref, s_lib) and np.array_equal(n_ref, n_lib)
    sl_ptr = sl.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    assert mla.lib().mla_max_parts(sl_ptr, len(sl), 16, 1, 0, 256, 3) == 3 + 2 + 3 + 3 + 1
    sched, ns, total = mla.get_mla_metadata_host(sl, 128, 1, num_cus=256)
    s_ref, n_ref = oracle.plan(sl, num_parts=256, fixed_overhead=4)
    assert np.array_equal(sched, s_ref) and np.array_equal(ns, n_ref)


UBSAN_HARNESS = r'''
#include <cstdint>
#include <cstdio>
#include <vector>
#include "mla_internal.h"
namespace mla {
int set_error(int code, const char*, ...) { return code; }
}
int main() {
  const int32_t lens[] = {2147483647, 100, 2147483584, 2147483583, 0, 1, 63, 64, 65};
  const int b = sizeof lens / sizeof lens[0];
  std::vector<int32_t> sched(4096 * 8), ns(b + 1);
  int parts = 0;
  for (int P : {1, 7, 256, 4096})
    for (int F : {0, 3, 8})
      if (mla::plan(lens, b, P, F, 0, sched.data(), 4096, ns.data(), &parts) != 0) return 2;
  for (int k : {1, 3, 64})
    if (mla::plan(lens, b, 1, 0, k, sched.data(), 4096, ns.data(), &parts) != 0) return 3;
  std::vector<int32_t> table(b * 64, 0);
  if (mla::plan(lens, b, 1, 0, 0, sched.data(), 4096, ns.data(), &parts) != 0) return 4;
  if (mla::attach_pages(sched.data(), parts, lens, b, table.data(), 64, 1) != 0 || sched[6] != 1) return 5;
  if (mla::plan(lens, b, 4096, 3, 0, sched.data(), 4096, ns.data(), &parts) != 0) return 6;
  if (mla::attach_pages(sched.data(), parts, lens, b, table.data(), 64, 1) == 0) return 7;   // pages past 64
  for (int L : {2147483647, 2147483584, 2147483583, 1, 0, -5})
    std::printf("%d ", mla::pages_of(L));
  std::printf("ok\n");
  return 0;
}
'''


def test_host_planner_under_undefined_behaviour_sanitizer(tmp_path):
    """The host planner (plain C++) built with g++ -fsanitize=undefined and run
    on lengths up to 2^31 - 1: no signed overflow or other undefined behaviour
    (the build traps on the first report)."""
    import shutil
    import subprocess
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    csrc = os.path.join(ROOT, "decode_attention_mla_amd", "csrc")
    src = tmp_path / "harness.cpp"
    src.write_text(UBSAN_HARNESS)
    exe = tmp_path / "harness"
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=undefined", "-fno-sanitize-recover=all",
           "-I", csrc, "-I", os.path.join(ROOT, "include"), str(src), os.path.join(csrc, "planner.cpp"), "-o", str(exe)]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0 and "runtime error" not in run.stderr, run.stdout + run.stderr
    assert run.stdout.split()[:6] == ["33554432", "33554431", "33554431", "1", "0", "0"], run.stdout
