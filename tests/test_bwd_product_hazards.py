"""The dK/dV kernel's inline-assembly matrix products keep their result
hazards by schedule (CPU only: compiles attn_bwd.hip to gfx950 assembly).

Stage 1 of the dK/dV kernel writes its S and dP products as inline assembly
(result in vector registers, the K or V operand in accumulation registers).
The compiler does not see those as matrix products, so it neither delays a
later access to their result registers nor accounts for their latency.  The
kernel's slot schedule keeps every such access away instead: a product's
result is accumulated into only by the next product of its own chain, and is
read by stage 2 of the next step, which starts at its fourth product slot.

This test reads the compiled code, follows its branches, and checks that on
every path at least four other matrix products issue between an
inline-assembly product and the first other instruction that reads or writes
its result registers.  A compiler or source change that moves such an access
closer fails here, on the CPU, before it can reach a GPU.  It also checks
that no compiler-generated instruction of the backward kernels touches M0,
which the inline-assembly copies set without the compiler preserving it.
"""

import heapq
import os
import re
import shutil
import subprocess

import pytest

from static_block_sparse_amd import build as B

MIN_PRODUCTS_BETWEEN = 4
KERNEL = r"_ZN6radial22radial_bwd_dkdv_kernel\w+"


def _regs(tok):
    m = re.match(r"v\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _parse(body):
    """Instructions of one function (op, args, from inline assembly) and its
    label positions."""
    ins, labels, in_asm = [], {}, False
    for line in body.splitlines():
        s = line.strip()
        m = re.match(r"^(\.LBB\w+):", s)
        if m:
            labels[m.group(1)] = len(ins)
            continue
        if s.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if s.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if not s or s.startswith((";", ".")) or s.endswith(":"):
            continue
        s = s.split(";")[0].strip()
        parts = s.split(None, 1)
        args = [a.strip() for a in parts[1].split(",")] if len(parts) > 1 else []
        ins.append((parts[0], args, in_asm))
    return ins, labels


def _successors(ins, labels, i):
    op, args, _ = ins[i]
    if op == "s_endpgm":
        return []
    if op == "s_branch":
        return [labels[args[0]]]
    if op.startswith("s_cbranch"):
        return [labels[args[0]], i + 1]
    return [i + 1] if i + 1 < len(ins) else []


def _fewest_products_before_access(ins, labels, i):
    """Fewest matrix products issued, over all paths, between the product at
    i and the first other instruction touching its result registers (None if
    none is reached).  An access by the next product of the same chain (the
    same registers as result and accumulator) continues the chain instead."""
    dst = _regs(ins[i][1][0])
    best = None
    seen = {}
    heap = [(0, s) for s in _successors(ins, labels, i)]
    while heap:
        cost, j = heapq.heappop(heap)
        if seen.get(j, 1 << 30) <= cost or (best is not None and cost >= best):
            continue
        seen[j] = cost
        op, args, _ = ins[j]
        touched = set().union(*(_regs(a) for a in args)) if args else set()
        if touched & dst:
            chain = (op.startswith("v_mfma") and len(args) > 3 and _regs(args[0]) == dst
                     and _regs(args[3]) == dst)
            if not chain:
                best = cost if best is None else min(best, cost)
            continue
        nxt = cost + (1 if op.startswith("v_mfma") else 0)
        for s in _successors(ins, labels, j):
            heapq.heappush(heap, (nxt, s))
    return best


@pytest.fixture(scope="module")
def bwd_assembly(tmp_path_factory):
    """attn_bwd.hip compiled for gfx950 as the build compiles it, as text."""
    if not shutil.which(B.HIPCC) and not os.path.exists(B.HIPCC):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "attn_bwd.s"
    cmd = [B.HIPCC, "-x", "hip", *B.DEVICE, *[f for f in B.COMMON if f != "-fPIC"],
           "--cuda-device-only", "-S", os.path.join(B.CSRC, "attn_bwd.hip"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    return out.read_text()


@pytest.fixture(scope="module")
def dkdv_assembly(bwd_assembly):
    funcs = re.findall(rf"^({KERNEL}):[^\n]*\n(.*?)^\.Lfunc_end", bwd_assembly, re.M | re.S)
    # every (D, T, token-exact) instantiation: (64, 64), (64, 128), (128, 128) x 2
    assert len(funcs) == 6, [f[0] for f in funcs]
    return funcs


def test_inline_assembly_products_are_far_from_their_readers(dkdv_assembly):
    for name, body in dkdv_assembly:
        ins, labels = _parse(body)
        asm_products = [i for i, (op, _, a) in enumerate(ins) if a and op.startswith("v_mfma")]
        assert asm_products, f"{name}: no inline-assembly products found (parser out of date?)"
        distances = [_fewest_products_before_access(ins, labels, i) for i in asm_products]
        reached = [d for d in distances if d is not None]
        assert reached, f"{name}: no access to any product's result found"
        assert min(reached) >= MIN_PRODUCTS_BETWEEN, (name, sorted(reached)[:8])


def test_hazard_scan_flags_a_close_reader():
    # the hazard scan itself, on a hand-written sequence: a vector read of the
    # result right after the product, or one product later, is caught; four
    # products later is not
    body_close = """
\t;;#ASMSTART
\tv_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], a[0:3], v[0:15]
\t;;#ASMEND
\tv_mfma_f32_32x32x16_bf16 a[16:31], v[20:23], v[24:27], a[16:31]
\tv_add_f32_e32 v40, v3, v41
\ts_endpgm
"""
    ins, labels = _parse(body_close)
    assert _fewest_products_before_access(ins, labels, 0) == 1
    body_chain = """
\t;;#ASMSTART
\tv_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], a[0:3], v[0:15]
\t;;#ASMEND
\t;;#ASMSTART
\tv_mfma_f32_32x32x16_bf16 v[0:15], v[20:23], a[4:7], v[0:15]
\t;;#ASMEND
""" + "\tv_mfma_f32_32x32x16_bf16 a[16:31], v[20:23], v[24:27], a[16:31]\n" * 4 + """
\tv_mul_f32_e32 v40, v3, v41
\ts_endpgm
"""
    ins, labels = _parse(body_chain)
    # the first product's next access is its own chain; the second's reader
    # comes four products later
    assert _fewest_products_before_access(ins, labels, 0) is None
    assert _fewest_products_before_access(ins, labels, 1) == 4
    # across a branch: the shorter path counts
    body_branch = """
\t;;#ASMSTART
\tv_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], a[0:3], v[0:15]
\t;;#ASMEND
\ts_cbranch_vccz .LBB0_2
""" + "\tv_mfma_f32_32x32x16_bf16 a[16:31], v[20:23], v[24:27], a[16:31]\n" * 6 + """
.LBB0_2:
\tv_mov_b32_e32 v5, 0
\ts_endpgm
"""
    ins, labels = _parse(body_branch)
    assert _fewest_products_before_access(ins, labels, 0) == 0


@pytest.fixture(scope="module")
def bwd_functions(bwd_assembly):
    funcs = re.findall(r"^(_ZN6radial\w+kernel\w+):[^\n]*\n(.*?)^\.Lfunc_end", bwd_assembly,
                       re.M | re.S)
    assert len(funcs) >= 20, len(funcs)
    return funcs


def test_m0_is_used_only_by_the_inline_assembly_copies(bwd_functions):
    # The copies issued from inline assembly set M0 and list it as clobbered;
    # M0 is reserved by the compiler, which does not promise to preserve it
    # across them.  So no compiler-generated instruction of these kernels may
    # touch M0 at all.
    for name, body in bwd_functions:
        in_asm, bad = False, []
        for line in body.splitlines():
            s = line.strip()
            if s.startswith(";;#ASMSTART"):
                in_asm = True
                continue
            if s.startswith(";;#ASMEND"):
                in_asm = False
                continue
            if not s or s.startswith((";", ".")):
                continue
            if not in_asm and re.search(r"\bm0\b", s.split(";")[0]):
                bad.append(s)
        assert not bad, (name, bad[:4])
