"""Properties of the gfx950 device code that the hardware needs and the
compiler cannot check (CPU test: hipcc cross-compiles the device assembly).

The 128-row kernel issues its MFMAs as inline assembly, so the compiler's
hazard recognizer does not see them:
  * a VALU instruction that writes a VGPR an MFMA then reads (A, B or C
    operand) needs two wait states before the MFMA (it would read the stale
    value otherwise);
  * a 16-register MFMA result must not overlap the same instruction's A or B
    operand.
Both are checked on every inline MFMA of every kernel.  Also recorded: the
per-lane scratch of each kernel (no split-KV kernel spills inside a page loop;
only the sparse forms of the 128-row kernel keep a few request-level values).
"""
import os
import re
import shutil
import subprocess

import pytest

from decode_attention_mla_amd import build

HIPCC = shutil.which("hipcc") or ("/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else None)
pytestmark = pytest.mark.skipif(HIPCC is None, reason="hipcc not available")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("isa") / "mla.s")
    flags = [f for f in build.HIP_FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [HIPCC, *flags, "-I", os.path.join(build.PKG_DIR, "..", "include"), "-S", "--offload-device-only",
           os.path.join(build.CSRC, "mla_decode.hip"), "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return open(out).read().split("\n")


def _regs(text):
    out = set()
    for m in re.finditer(r"\b([va])\[(\d+):(\d+)\]", text):
        out |= {(m.group(1), r) for r in range(int(m.group(2)), int(m.group(3)) + 1)}
    for m in re.finditer(r"\b([va])(\d+)\b", text):
        out.add((m.group(1), int(m.group(2))))
    return out


def _inline_mfmas(lines):
    """(kernel, line index, instruction) of every MFMA inside inline assembly."""
    kern, inside = None, False
    for i, line in enumerate(lines):
        if re.match(r"^_Z\S+:", line):
            kern = line.split(":")[0]
        t = line.strip()
        if t.startswith(";;#ASMSTART"):
            inside = True
        elif t.startswith(";;#ASMEND"):
            inside = False
        elif inside and t.startswith("v_mfma"):
            yield kern, i, t


def test_inline_mfmas_present(asm):
    kernels = {k for k, _, _ in _inline_mfmas(asm)}
    assert sum("splitkv_wide_kernel" in k for k in kernels) == 8, kernels


def test_no_valu_write_feeds_inline_mfma(asm):
    bad = []
    for kern, i, ins in _inline_mfmas(asm):
        srcs = _regs(",".join(ins.split(None, 1)[1].split(",")[1:]))
        k, ws = i - 1, 0
        while k >= 0 and ws < 2:
            u = asm[k].strip()
            k -= 1
            if not u or u.startswith(";") or u.startswith("."):
                continue
            m = re.match(r"s_nop\s+(\d+)", u)
            if m:
                ws += int(m.group(1)) + 1
                continue
            ws += 1
            if u.startswith("v_") and not u.startswith("v_mfma"):
                parts = u.split(None, 1)
                if len(parts) > 1 and _regs(parts[1].split(",")[0]) & srcs:
                    bad.append((kern[:60], u, ins))
    assert not bad, bad[:5]


def test_inline_mfma_result_does_not_overlap_sources(asm):
    bad = []
    for kern, _, ins in _inline_mfmas(asm):
        ops = [o.strip() for o in ins.split(None, 1)[1].split(",")]
        if _regs(ops[0]) & (_regs(ops[1]) | _regs(ops[2])):
            bad.append((kern[:60], ins))
    assert not bad, bad[:5]


def test_barriers_with_reads_in_flight_publish_every_write(asm):
    """A barrier that waits for lgkmcnt(N) with N > 0 lets the wave's last N
    LDS operations stay in flight: they must all be reads, so that every LDS
    write the barrier publishes is older than them (LDS operations complete in
    order)."""
    found = 0
    for i, line in enumerate(asm):
        m = re.match(r"\s*s_waitcnt lgkmcnt\((\d+)\)\s*$", line)
        if not m or int(m.group(1)) == 0:
            continue
        nxt = [t.strip() for t in asm[i + 1:i + 4] if t.strip() and not t.strip().startswith(";")]
        if not nxt or not nxt[0].startswith("s_barrier"):
            continue
        n, k, last = int(m.group(1)), i - 1, []
        while k >= 0 and len(last) < n:
            t = asm[k].strip()
            k -= 1
            if t.startswith("ds_"):
                last.append(t)
            if re.match(r"^_Z\S+:", t):
                break
        found += 1
        assert len(last) == n and all(t.startswith("ds_read") for t in last), last
    assert found > 0


def test_no_scratch_access_in_a_page_loop(asm):
    """Spilled values, where a kernel has any, are read outside the page loop
    (the deepest loop that issues MFMAs)."""
    kern, depth, blocks = None, 0, {}
    for line in asm:
        m = re.match(r"^(_Z\S+):", line)
        if m:
            kern, depth = m.group(1), 0
            continue
        if kern is None or "splitkv" not in kern:
            continue
        t = line.strip()
        if t.startswith(".LBB") or t.startswith("; %bb"):
            d = re.search(r"Depth=(\d+)", t)
            depth = int(d.group(1)) if d else 0
        k = blocks.setdefault(kern, {"mfma": 0, "scratch": []})
        if t.startswith("v_mfma"):
            k["mfma"] = max(k["mfma"], depth)
        elif t.startswith("scratch_"):
            k["scratch"].append((depth, t))
    assert blocks
    bad = [(n[:60], d, t) for n, k in blocks.items() for d, t in k["scratch"] if d >= k["mfma"]]
    assert not bad, bad[:5]


def test_scratch_per_kernel(asm):
    text = "\n".join(asm)
    sizes = dict(re.findall(r"\.name:\s+(\S+)\n\s+\.private_segment_fixed_size:\s+(\d+)", text))
    assert sizes, "no kernel metadata found"
    for name, size in sizes.items():
        size = int(size)
        if re.search(r"splitkv_wide_kernelILb[01]ELb1E", name):
            assert size <= 48, (name, size)   # sparse 128-row kernels: request- and attempt-level values only
        else:
            assert size == 0, (name, size)
