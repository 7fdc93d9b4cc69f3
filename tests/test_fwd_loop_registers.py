"""The forward kernel's chunk loop runs without register spills (CPU only:
compiles attn_fwd.hip to gfx950 assembly).

With query tiles in triples, three waves share each SIMD and every wave has
168 registers, which the loop uses almost entirely (O accumulator, Q
operands, S, P and the read offsets).  Small source changes have made the
compiler spill there: the bf16 probabilities sunk past the chunk check's
branch, the tail mask words computed inside the chunk, the redo flag held as
an integer.  A spill inside the loop reloads a register from scratch memory
on every chunk and makes the reload wait for the chunk copies in flight.
This test compiles the kernel the way the build does and checks that no
scratch access (and no scalar spill to vector lanes) sits inside a loop of
any triple instantiation, so such a change is caught on the CPU.
"""

import os
import re
import shutil
import subprocess

import pytest

from static_block_sparse_amd import build as B

TRIPLE = r"_ZN6radial17radial_fwd_kernelILi(\d+)ELi(\d+)ELb([01])ELi3E\w*"


@pytest.fixture(scope="module")
def fwd_assembly(tmp_path_factory):
    if not shutil.which(B.HIPCC) and not os.path.exists(B.HIPCC):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "attn_fwd.s"
    cmd = [B.HIPCC, "-x", "hip", *B.DEVICE, *[f for f in B.COMMON if f != "-fPIC"],
           "--cuda-device-only", "-S", os.path.join(B.CSRC, "attn_fwd.hip"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    return out.read_text()


def _loop_lines(body):
    """Instruction lines of the blocks the compiler marks as inside a loop."""
    inside, out = False, []
    for line in body.splitlines():
        if line.startswith(".LBB") or line.startswith("; %bb"):
            inside = "Loop" in line
            continue
        s = line.strip()
        if inside and s and not s.startswith((";", ".")):
            out.append(s)
    return out


def test_triple_chunk_loops_do_not_spill(fwd_assembly):
    funcs = re.findall(rf"^({TRIPLE}):[^\n]*\n(.*?)^\.Lfunc_end", fwd_assembly, re.M | re.S)
    # (D, T) in (64, 64), (64, 128), (128, 128), tile and token-exact mode
    assert len(funcs) == 6, [f[0][:60] for f in funcs]
    for f in funcs:
        name, body = f[0], f[-1]
        loop = _loop_lines(body)
        assert len(loop) > 200, f"{name}: chunk loop not found"
        assert sum(l.startswith("v_mfma") for l in loop) >= 32, name
        spills = [l for l in loop if l.startswith("scratch_") or l.startswith("v_writelane")]
        assert not spills, (name, spills[:4])
