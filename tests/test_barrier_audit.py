"""Static audit of the built device code: no workgroup barrier is reached
while this wave's global-to-LDS tile copies may still be in flight.

Kernels stage K, V, Q and dO tiles with buffer loads that write LDS
directly.  A barrier does not wait for those copies, so each wave must wait
for its own (s_waitcnt vmcnt(0)) before the barrier that hands the tile to
the other waves; otherwise another wave can read a tile that has not
landed.  This test compiles the sources that issue such copies to gfx950
assembly and runs a forward data-flow pass over each kernel's control-flow
graph (state: a copy issued and not yet waited for), failing on any
s_barrier reached in that state.  CPU only: it needs hipcc, not a GPU."""
import os
import re
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_attention_18_amd", "csrc")
SOURCES = ["forward.hip", "fp8.hip", "backward.hip", "scores.hip"]

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not found")

COPY = re.compile(r"^\s*buffer_load\w*\b.*\blds\b")
FULL_WAIT = re.compile(r"^\s*s_waitcnt\b.*\bvmcnt\(0\)")
BARRIER = re.compile(r"^\s*s_barrier\b")
LABEL = re.compile(r"^(\.LBB\w+):")
BRANCH = re.compile(r"^\s*(s_branch|s_cbranch_\w+)\s+(\.LBB\w+)")
FUNC = re.compile(r"^(_Z\w+):")


def _compile(src, outdir):
    out = os.path.join(outdir, src + ".s")
    cmd = ["hipcc", "-x", "hip", "-O3", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC, "--cuda-device-only",
           "-S", os.path.join(CSRC, src), "-o", out]
    subprocess.run(cmd, check=True, capture_output=True)
    return out


def _kernels(lines):
    """(name, body lines) of every function in an assembly listing."""
    cur, body = None, []
    for ln in lines:
        m = FUNC.match(ln)
        if m:
            if cur:
                yield cur, body
            cur, body = m.group(1), []
        elif cur:
            if ln.strip().startswith(".Lfunc_end"):
                yield cur, body
                cur, body = None, []
            else:
                body.append(ln)
    if cur:
        yield cur, body


def _blocks(body):
    """Basic blocks: (label, instructions, successor labels)."""
    blocks, label, ins = [], "<entry>", []
    def close(next_label):
        succ, fall = [], True
        for x in ins:
            m = BRANCH.match(x)
            if m:
                succ.append(m.group(2))
                if m.group(1) == "s_branch":
                    fall = False
        if ins and re.match(r"^\s*s_endpgm\b", ins[-1]):
            fall = False
        blocks.append([label, list(ins), succ, fall, next_label])
    for ln in body:
        m = LABEL.match(ln)
        if m:
            close(m.group(1))
            label, ins = m.group(1), []
            continue
        if ln.strip() and not ln.strip().startswith((";", ".")):
            ins.append(ln)
            if BRANCH.match(ln) or re.match(r"^\s*s_endpgm\b", ln):
                # a block ends at a branch; the rest is a fall-through block
                close(None)
                blocks[-1][4] = f"{label}+{len(blocks)}"
                label, ins = blocks[-1][4], []
    close(None)
    return blocks


def _violations(body):
    blocks = _blocks(body)
    index = {b[0]: i for i, b in enumerate(blocks)}
    succs = []
    for i, (label, ins, targets, fall, nxt) in enumerate(blocks):
        s = [index[t] for t in targets if t in index]
        if fall and i + 1 < len(blocks):
            s.append(i + 1)
        succs.append(s)
    pending_in = [False] * len(blocks)
    work = list(range(len(blocks)))
    bad = set()
    while work:
        i = work.pop()
        p = pending_in[i]
        for ln in blocks[i][1]:
            if COPY.match(ln):
                p = True
            elif FULL_WAIT.match(ln):
                p = False
            elif BARRIER.match(ln) and p:
                bad.add(blocks[i][0])
        for j in succs[i]:
            if p and not pending_in[j]:
                pending_in[j] = True
                work.append(j)
    return sorted(bad)


def test_no_barrier_with_tile_copies_in_flight():
    with tempfile.TemporaryDirectory() as tmp:
        with ThreadPoolExecutor(max_workers=4) as ex:
            outs = list(ex.map(lambda s: _compile(s, tmp), SOURCES))
        checked, problems = 0, []
        for out in outs:
            lines = open(out).read().split("\n")
            for name, body in _kernels(lines):
                if not any(COPY.match(ln) for ln in body):
                    continue
                checked += 1
                v = _violations(body)
                if v:
                    problems.append(f"{os.path.basename(out)} {name}: barrier with copies in flight in {v}")
    assert checked >= 30, f"only {checked} kernels with tile copies found"
    assert not problems, "\n".join(problems)
