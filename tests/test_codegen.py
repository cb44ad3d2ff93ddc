"""Code generation of the attention kernel for gfx950 (CPU only: hipcc cross-compiles).

The ping-pong loop relies on its own waits: a wavefront issues its direct global->LDS
loads at the end of its VALU phase and waits for them (all vector-memory counters at
zero) at the end of its next VALU phase, two periods later; in its MFMA phase in between
it reads only ring slots whose loads completed earlier.  The compiler cannot see that a
wavefront alternates between the two phases (the group condition is per wavefront), and
where its bookkeeping of direct-to-LDS loads loses track it inserts a bare
`s_waitcnt vmcnt(0)` in the MFMA phase, which stalls the matrix core on loads issued just
before the barrier.  Measured on MI355X: removing the one such wait of the 128-row loop
(once every four periods) made the 1024x1024 text-to-image denoising step 1.5-1.9%
faster.  This test keeps the steady loops of the bf16 kernels free of it."""
from __future__ import annotations

import os
import re
import shutil
import subprocess

import pytest

from block_causal_attention_qi_amd import build

SRC = os.path.join(build.CSRC, "attn_fwd.hip")


def _asm(tmp_path):
    try:
        hipcc = build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    out = str(tmp_path / "attn_fwd.s")
    flags = [f for f in build.flags() if f not in ("-shared", "-fPIC")]
    res = subprocess.run([hipcc] + flags + ["--cuda-device-only", "-S", SRC, "-o", out],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return open(out).read().splitlines()


def _function(lines, d, src):
    """Body of attn_pp_kernel<d, src> (from its label to .Lfunc_end)."""
    pat = re.compile(r"^(_Z\S*attn_pp_kernelILi%dELi%dEE\S*):" % (d, src))
    start = next(i for i, l in enumerate(lines) if pat.match(l))
    end = next(i for i in range(start, len(lines)) if lines[i].startswith(".Lfunc_end"))
    return lines[start:end]


def _steady_loops(body, mfma_per_iter):
    """(first, last) line of every loop (a label and a later branch back to it) whose body
    holds exactly the MFMAs of four key tiles."""
    labels = {}
    for i, l in enumerate(body):
        m = re.match(r"^(\.LBB\d+_\d+):", l)
        if m:
            labels[m.group(1)] = i
    loops = []
    for i, l in enumerate(body):
        m = re.search(r"\bs_(?:cbranch_\w+|branch)\s+(\.LBB\d+_\d+)\b", l)
        if m and m.group(1) in labels and labels[m.group(1)] < i:
            a = labels[m.group(1)]
            if sum("v_mfma" in x for x in body[a:i + 1]) == mfma_per_iter:
                loops.append((a, i))
    return loops


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_bf16_steady_loops_hold_no_bare_load_wait(tmp_path):
    lines = _asm(tmp_path)
    d = 128
    mfma_per_iter = 4 * (2 * d // 16 + 4 * d // 32)   # QK 2 x D/16, PV 4 x D/32 per tile
    for src, what in ((0, "one source (prefix and full calls)"), (1, "bf16 cache (denoising)")):
        body = _function(lines, d, src)
        loops = _steady_loops(body, mfma_per_iter)
        # one steady loop each for row tiles of 256 rows and of at most 128 rows
        assert len(loops) >= 2, (what, loops)
        for a, b in loops:
            bare = [body[i].strip() for i in range(a, b + 1)
                    if re.match(r"\s*s_waitcnt\s+vmcnt\(0\)\s*$", body[i])]
            assert not bare, "%s: %d bare vmcnt(0) waits in the loop at lines %d-%d" % (
                what, len(bare), a, b)
