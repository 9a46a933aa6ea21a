"""The hand-counted vector-memory waits of the tiled MFMA kernels hold in the
code the compiler emits (gfx950 assembly, no GPU needed).

Vector-memory operations of a wave complete in issue order, so a barrier that
waits with vmcnt(N) leaves exactly the N youngest in flight.  The kernels count
those on purpose: LDS copies of later blocks (buffer loads with the LDS bit)
and, last, the L2 prefetch of a block's weight lines (one dword into a
register).  That is exact only while the emitted order is the written one, on
the fall-through path and on a loop's back edge alike.  The loaded row pointers
are restrict-qualified, so the compiler is free to move a plain load (a variant
that staged token rows through registers had its loads sunk past a barrier
that way).  These tests compile tiled_gemm.hip and backward.hip to assembly
and check, before every counted barrier (vmcnt(N) with N > 0, then s_barrier)
of every tiled and backward GEMM kernel: the N youngest vector-memory
instructions are LDS copies, except that the youngest may be the prefetch, and
for vmcnt(1) it must be.
"""
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "sparse_moe_transformer_way_amd"))
import build as B  # noqa: E402

VMEM = re.compile(r"^\s*(buffer|global|flat)_(load|store|atomic)\w*")
PREFETCH = re.compile(r"^\s*buffer_load_dword\s+v\d+,(?!.*\blds\b)")  # one dword into a VGPR, no LDS bit
LDS_COPY = re.compile(r"^\s*buffer_load_dword\w*\s.*\blds\s*$")       # a copy straight into LDS
LABEL = re.compile(r"^(\.LBB\w+):")
BRANCH = re.compile(r"^\s*s_cbranch_\w+\s+(\.LBB\w+)|^\s*s_branch\s+(\.LBB\w+)")


def _instructions(text):
    out = []
    for line in text.splitlines():
        code = line.split(";", 1)[0].rstrip()
        if code.strip():
            out.append(code)
    return out


def _kernels(asm, kernel="tiled_kernel"):
    """{symbol: ([instruction lines], {loop header labels})} for each instantiation of `kernel`."""
    kernels = {}
    for m in re.finditer(r"^(_ZN\w*" + kernel + r"\w*):.*?$(.*?)^\.Lfunc_end\d+:", asm, re.M | re.S):
        headers = set(re.findall(r"^(\.LBB\w+):\s*;.*Loop Header", m.group(2), re.M))
        kernels[m.group(1)] = (_instructions(m.group(2)), headers)
    return kernels


def _asm(tmp_path_factory, name):
    out = tmp_path_factory.mktemp("asm") / (name + ".s")
    src = os.path.join(B.CSRC, name + ".hip")
    r = subprocess.run([B.hipcc(), *B.HIPCC_FLAGS, "--cuda-device-only", "-S", src, "-o", str(out)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


@pytest.fixture(scope="module")
def tiled_asm(tmp_path_factory):
    return _asm(tmp_path_factory, "tiled_gemm")


@pytest.fixture(scope="module")
def backward_asm(tmp_path_factory):
    return _asm(tmp_path_factory, "backward")


def _window_ok(window, n):
    """The n youngest vector-memory instructions (oldest first): LDS copies,
    the youngest possibly the prefetch (and for n == 1 necessarily)."""
    if len(window) < n:
        return False
    *older, youngest = window[-n:]
    if n == 1:
        return PREFETCH.match(youngest) is not None
    return all(LDS_COPY.match(w) for w in older) and (LDS_COPY.match(youngest) or PREFETCH.match(youngest))


def _check(lines, headers):
    """Returns (number of counted barriers, violations)."""
    labels = {LABEL.match(l).group(1): i for i, l in enumerate(lines) if LABEL.match(l)}
    before = []  # line index -> vector-memory instructions before it, in textual order
    seen = []
    for l in lines:
        before.append(list(seen[-64:]))
        if VMEM.match(l):
            seen.append(l.strip())
    bad, count = [], 0
    for i, l in enumerate(lines):
        m = re.match(r"^\s*s_waitcnt\b.*\bvmcnt\((\d+)\)", l)
        if not (m and int(m.group(1)) > 0 and i + 1 < len(lines) and lines[i + 1].strip().startswith("s_barrier")):
            continue
        n = int(m.group(1))
        count += 1
        if not _window_ok(before[i], n):
            bad.append((i, f"fall-through vmcnt({n})", before[i][-n:]))
        # a loop header that leads straight to this barrier: every back edge to it must end the same way
        head = next((k for k in range(i - 1, -1, -1) if LABEL.match(lines[k]) or BRANCH.match(lines[k])), None)
        if head is not None and LABEL.match(lines[head]) and LABEL.match(lines[head]).group(1) in headers:
            target = LABEL.match(lines[head]).group(1)
            for j in range(head + 1, len(lines)):
                b = BRANCH.match(lines[j])
                if b and (b.group(1) or b.group(2)) == target and not _window_ok(before[j], n):
                    bad.append((j, f"back edge vmcnt({n})", before[j][-n:]))
    return count, bad


def test_prefetch_is_the_last_load_before_counted_barriers(tiled_asm):
    kernels = _kernels(tiled_asm)
    assert any("ILb0E" in k for k in kernels) and any("ILb1E" in k for k in kernels), list(kernels)
    total = 0
    for name, (lines, headers) in kernels.items():
        count, bad = _check(lines, headers)
        total += count
        assert not bad, (name, bad[:5])
    # the down projection and the prefetching gate/up tiles both have such barriers
    assert total > 0


def test_backward_gemm_counted_barriers(backward_asm):
    """The backward GEMM's ring of four 32-k stages: each stage's barrier leaves
    the copies of the later stages in flight, and only those."""
    kernels = _kernels(backward_asm, "bwd_gemm_kernel")
    assert len(kernels) >= 3, list(kernels)
    for name, (lines, headers) in kernels.items():
        count, bad = _check(lines, headers)
        assert count > 0 and not bad, (name, count, bad[:5])


GOOD = """
	buffer_load_dwordx4 v1, s[4:7], s8 offen lds
	buffer_load_dword v2, v59, s[4:7], s70 offen
.LBB0_5:                                ; =>This Inner Loop Header: Depth=1
	s_waitcnt vmcnt(1) lgkmcnt(0)
	s_barrier
	buffer_load_dwordx4 v1, s[4:7], s8 offen lds
	buffer_load_dword v3, v59, s[4:7], s70 offen
	s_cbranch_scc1 .LBB0_5
	s_endpgm
"""


def test_checker_flags_a_load_moved_past_the_barrier():
    """The checker itself: the order above passes; a copy issued after the
    prefetch on the back edge, or no prefetch before the loop, fails."""
    def run(text):
        m = {"k": (_instructions(text), set(re.findall(r"^(\.LBB\w+):\s*;.*Loop Header", text, re.M)))}
        return _check(*m["k"])
    assert run(GOOD) == (1, [])
    back = GOOD.replace("\tbuffer_load_dword v3, v59, s[4:7], s70 offen\n",
                        "\tbuffer_load_dword v3, v59, s[4:7], s70 offen\n\tbuffer_load_dwordx4 v1, s[4:7], s9 offen lds\n")
    assert [b[1] for b in run(back)[1]] == ["back edge vmcnt(1)"]
    entry = GOOD.replace("\tbuffer_load_dword v2, v59, s[4:7], s70 offen\n", "")
    assert [b[1] for b in run(entry)[1]] == ["fall-through vmcnt(1)"]
    # vmcnt(3): the 3 youngest are two copies and the prefetch; a register load among them fails
    three = GOOD.replace("vmcnt(1)", "vmcnt(3)").replace(
        "\tbuffer_load_dword v2, v59, s[4:7], s70 offen\n",
        "\tbuffer_load_dwordx4 v1, s[4:7], s9 offen lds\n\tbuffer_load_dword v2, v59, s[4:7], s70 offen\n").replace(
        "\tbuffer_load_dword v3, v59, s[4:7], s70 offen\n",
        "\tbuffer_load_dwordx4 v1, s[4:7], s9 offen lds\n\tbuffer_load_dword v3, v59, s[4:7], s70 offen\n")
    assert run(three) == (1, [])
    reg = three.replace("\tbuffer_load_dwordx4 v1, s[4:7], s9 offen lds\n\tbuffer_load_dword v2,",
                        "\tbuffer_load_dwordx4 v[8:11], v5, s[0:3], s9 offen\n\tbuffer_load_dword v2,")
    assert [b[1] for b in run(reg)[1]] == ["fall-through vmcnt(3)"]
