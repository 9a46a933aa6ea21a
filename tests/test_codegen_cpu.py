"""The hand-counted vector-memory waits of the tiled MFMA kernels hold in the
code the compiler emits (gfx950 assembly, no GPU needed).

Where a tile prefetches its weight lines into L2, the barrier before the second
stage of a block waits with vmcnt(1): vector-memory operations of a wave
complete in issue order, and the one operation allowed to stay in flight is
meant to be that prefetch, issued after the block's LDS copies.  That is exact
only while the prefetch is the wave's last vector-memory instruction before the
barrier, on the fall-through path and on a loop's back edge alike.  The loaded
row pointers are restrict-qualified, so the compiler is free to move such a
load (a variant that staged token rows through registers had its loads sunk
past a barrier that way).  This test compiles tiled_gemm.hip to assembly and
checks the order in every tiled kernel.
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
PREFETCH = re.compile(r"^\s*buffer_load_dword\s+v\d+,")  # one dword into a VGPR, no LDS bit
LABEL = re.compile(r"^(\.LBB\w+):")
BRANCH = re.compile(r"^\s*s_cbranch_\w+\s+(\.LBB\w+)|^\s*s_branch\s+(\.LBB\w+)")


def _instructions(text):
    out = []
    for line in text.splitlines():
        code = line.split(";", 1)[0].rstrip()
        if code.strip():
            out.append(code)
    return out


def _kernels(asm):
    """{symbol: ([instruction lines], {loop header labels})} for each tiled_kernel instantiation."""
    kernels = {}
    for m in re.finditer(r"^(_ZN\w*tiled_kernel\w*):.*?$(.*?)^\.Lfunc_end\d+:", asm, re.M | re.S):
        headers = set(re.findall(r"^(\.LBB\w+):\s*;.*Loop Header", m.group(2), re.M))
        kernels[m.group(1)] = (_instructions(m.group(2)), headers)
    return kernels


@pytest.fixture(scope="module")
def tiled_asm(tmp_path_factory):
    out = tmp_path_factory.mktemp("asm") / "tiled_gemm.s"
    src = os.path.join(B.CSRC, "tiled_gemm.hip")
    r = subprocess.run([B.hipcc(), *B.HIPCC_FLAGS, "--cuda-device-only", "-S", src, "-o", str(out)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def _check(lines, headers):
    """Returns (number of vmcnt(1) barriers, violations)."""
    labels = {LABEL.match(l).group(1): i for i, l in enumerate(lines) if LABEL.match(l)}
    last_at = []  # line index -> latest vector-memory instruction before it, in textual order
    last_vmem = None
    for l in lines:
        last_at.append(last_vmem)
        if VMEM.match(l):
            last_vmem = l.strip()
    bad, count = [], 0
    for i, l in enumerate(lines):
        last_vmem = last_at[i]
        if re.match(r"^\s*s_waitcnt\b.*\bvmcnt\(1\)", l) and i + 1 < len(lines) and \
                lines[i + 1].strip().startswith("s_barrier"):
            count += 1
            if last_vmem is None or not PREFETCH.match(last_vmem):
                bad.append((i, "fall-through", last_vmem))
            # a loop whose header leads to this barrier: its back edge must end with the prefetch too
            for j in range(i + 1, len(lines)):
                b = BRANCH.match(lines[j])
                if not b:
                    continue
                target = b.group(1) or b.group(2)
                if target in headers and labels[target] <= i:
                    prev = last_at[j]
                    if prev is None or not PREFETCH.match(prev):
                        bad.append((j, "back edge", prev))
                    break
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
    assert [b[1] for b in run(back)[1]] == ["back edge"]
    entry = GOOD.replace("\tbuffer_load_dword v2, v59, s[4:7], s70 offen\n", "")
    assert [b[1] for b in run(entry)[1]] == ["fall-through"]
