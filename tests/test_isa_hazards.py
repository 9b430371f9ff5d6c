"""Static checks of hazards that the compiler does not cover in inline assembly.

1. Matrix-core hazards in the latent decode kernel (2. LDS-DMA SGPR operands and 3. serialized loads, in every kernel, further down).

The latent kernel issues its v_mfma instructions from inline assembly (to pin
the output accumulators to the accumulation registers), so the compiler's
hazard recognizer does not see them.  This test compiles the kernel source
to gfx950 assembly with the library's own flags and checks, in straight-line
code, the two hazards the source relies on avoiding:

* a VALU write of a register that a following v_mfma reads (A, B or C)
  needs 2 wait states in between; the check asks for 3;
* a v_mfma result may be read or written by anything other than the next
  product of the same chain (same C and destination) only after the product
  has drained; the check asks for 24 wait states, above the pass count plus
  write-back latency of the 32x32x16 bf16 product.

Wait states are counted as one per instruction, s_nop N as N + 1.  The scan
follows the control flow: from each product forward along every fall-through
and branch edge (s_branch has no fall-through; s_endpgm ends a path), and
backward along every edge into the product, so a hazard that spans a branch
(a result read on one side of a uniform if, say) is seen.

2. The LDS-DMA loads of every kernel (global_load_lds, issued from inline
assembly with an SGPR base): a vector memory instruction may read an SGPR
only 5 wait states after a VALU instruction wrote it.  The compiler inserts
that for its own loads, not inside asm; it bites when register pressure makes
the compiler spill a base pointer to a VGPR lane and reload it with
v_readlane right before the load (a stale base is an out-of-bounds address).
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "paged_kv_cache_58_amd", "csrc", "latent_decode.hip")
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

VALU_TO_MFMA = 3
MFMA_DRAIN = 24

_REG = re.compile(r"\b([va])(?:\[(\d+):(\d+)\]|(\d+)(?!\w))")


def _regs(text: str) -> set[tuple[str, int]]:
    out = set()
    for m in _REG.finditer(text):
        f = m.group(1)
        if m.group(4) is not None:
            out.add((f, int(m.group(4))))
        else:
            out.update((f, i) for i in range(int(m.group(2)), int(m.group(3)) + 1))
    return out


def _is_branch(mn: str) -> bool:
    return mn.startswith("s_cbranch") or mn == "s_branch"


def parse(lines) -> tuple[list[tuple[str, str]], list[list[int]]]:
    """Instructions of one function body (a list of assembly lines) and the
    successors of each: the next instruction unless it is an unconditional
    branch or ends the program, plus the target of a branch."""
    instrs: list[tuple[str, str]] = []
    labels: dict[str, int] = {}
    for line in lines:
        s = line.split(";", 1)[0].strip()
        if not s:
            continue
        if s.endswith(":"):
            labels[s[:-1]] = len(instrs)
            continue
        if s.startswith("."):
            continue
        parts = s.split(None, 1)
        instrs.append((parts[0], parts[1] if len(parts) > 1 else ""))
    succ: list[list[int]] = []
    for i, (mn, ops) in enumerate(instrs):
        nxt = []
        if mn not in ("s_branch", "s_endpgm", "s_setpc_b64") and i + 1 < len(instrs):
            nxt.append(i + 1)
        if _is_branch(mn):
            target = ops.split(",")[0].strip()
            if target in labels and labels[target] < len(instrs):
                nxt.append(labels[target])
        succ.append(nxt)
    return instrs, succ


def _preds(succ: list[list[int]]) -> list[list[int]]:
    pred: list[list[int]] = [[] for _ in succ]
    for i, nx in enumerate(succ):
        for j in nx:
            pred[j].append(i)
    return pred


def _functions(asm: str, kernel_prefix: str) -> list[list[str]]:
    """Body lines of every function whose name starts with kernel_prefix."""
    out = []
    for m in re.finditer(r"^(_Z\w+):", asm, re.M):
        if m.group(1).startswith(kernel_prefix):
            out.append(asm[m.end():asm.find(".Lfunc_end", m.end())].splitlines())
    return out


def _wait_states(mn: str, ops: str) -> int:
    if mn == "s_nop":
        return int(ops.strip(), 0) + 1
    return 1


def _is_valu(mn: str) -> bool:
    return mn.startswith("v_") and not mn.startswith("v_mfma")


def _dst(ops: str) -> set[tuple[str, int]]:
    first = ops.split(",", 1)[0]
    return _regs(first)


def _walk(start: list[int], edges: list[list[int]], budget: int, visit) -> None:
    """Every instruction reachable from `start` along `edges` with fewer than
    `budget` wait states between it and the origin; visit(j, ws) returns
    False to stop the path there.  Each instruction is entered again only by
    a path with fewer wait states than before."""
    best: dict[int, int] = {}
    stack = [(j, 0) for j in start]
    while stack:
        j, ws = stack.pop()
        if ws >= budget or best.get(j, budget) <= ws:
            continue
        best[j] = ws
        if visit(j, ws):
            stack.extend((k, ws + visit.cost(j)) for k in edges[j])


def check(lines) -> list[str]:
    """Matrix-core hazards in one function body (assembly lines)."""
    instrs, succ = parse(lines)
    pred = _preds(succ)
    problems = []
    for i, (mn, ops) in enumerate(instrs):
        if not mn.startswith("v_mfma"):
            continue
        fields = [f.strip() for f in ops.split(",")]
        dst, srcs = _regs(fields[0]), set()
        for f in fields[1:4]:
            srcs |= _regs(f)

        # VALU writes shortly before the product, along every path into it
        def back(j, ws):
            pm, pops = instrs[j]
            if _is_valu(pm) and _dst(pops) & srcs:
                problems.append(f"{pm} {pops} -> {mn} {ops} after {ws} wait states")
            return True
        back.cost = lambda j: _wait_states(*instrs[j])
        _walk(pred[i], pred, VALU_TO_MFMA, back)

        # uses of the result before it has drained, along every path out of it
        def fwd(j, ws):
            nm, nops = instrs[j]
            if nm.startswith("v_mfma"):
                nf = [f.strip() for f in nops.split(",")]
                same_chain = _regs(nf[0]) == dst and _regs(nf[3]) == dst
                touches = (_regs(nf[0]) | _regs(nf[1]) | _regs(nf[2]) | _regs(nf[3])) & dst
                if touches and not same_chain:
                    problems.append(f"{mn} {ops} -> {nm} {nops} after {ws} wait states")
                if same_chain:
                    return False  # the chain's next link takes over the result
            elif _regs(nops) & dst:
                problems.append(f"{mn} {ops} -> {nm} {nops} after {ws} wait states")
            return True
        fwd.cost = lambda j: _wait_states(*instrs[j])
        _walk(succ[i], succ, MFMA_DRAIN, fwd)
    return problems


@pytest.fixture(scope="module")
def latent_asm(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    out = tmp_path_factory.mktemp("isa") / "latent.s"
    cmd = [HIPCC, "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-O3", "-std=c++17", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.dirname(SRC), "-x", "hip", "-S", "--cuda-device-only", SRC,
           "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return out.read_text()


LATENT = "_ZN2pa12_GLOBAL__N_123latent_partition_kernel"


def test_latent_kernel_has_products(latent_asm):
    fns = _functions(latent_asm, LATENT)
    assert len(fns) == 3
    n = sum(1 for f in fns for mn, _ in parse(f)[0] if mn.startswith("v_mfma"))
    # three instantiations (1, 2 and 4 head tiles): per unit 36 / KS score
    # products (the wave's share of its tile's contraction, KS = 4 / tiles)
    # and 8 value products per head tile
    assert n >= (9 + 8) + (18 + 16) + (36 + 32)


def test_latent_kernel_mfma_hazards(latent_asm):
    problems = []
    for body in _functions(latent_asm, LATENT):
        problems += check(body)
    assert not problems, "\n".join(problems[:20])


def test_checker_catches_planted_hazards():
    """The checker itself flags a VALU write right before a product and a
    read of a product's result before it drains, also across a branch, and
    passes a fenced chain."""
    assert check(["v_mov_b32 v4, 0", "v_mfma_f32_32x32x16_bf16 v[10:25], v[2:5], v[6:9], 0"])
    assert check(["v_mfma_f32_32x32x16_bf16 v[10:25], v[2:5], v[6:9], 0",
                  "v_add_f32_e32 v30, v10, v11"])
    ok = ["v_mfma_f32_32x32x16_bf16 v[10:25], v[2:5], v[6:9], 0",
          "ds_read_b128 v[2:5], v40",
          "v_mfma_f32_32x32x16_bf16 v[10:25], v[26:29], v[6:9], v[10:25]",
          "s_nop 7", "s_nop 7", "s_nop 7", "s_nop 7",
          "v_add_f32_e32 v30, v10, v11"]
    assert not check(ok)
    # the read sits behind a taken branch: a block-local scan would miss it
    cross = ["v_mfma_f32_32x32x16_bf16 a[0:15], v[2:5], v[6:9], a[0:15]",
             "s_cbranch_scc1 .LBB0_2",
             "s_nop 7", "s_nop 7", "s_nop 7", "s_nop 7",
             ".LBB0_2:",
             "v_accvgpr_read_b32 v30, a3"]
    assert check(cross)
    # ... and one on the fall-through side of an unconditional branch is not
    # reachable from the product
    dead = ["v_mfma_f32_32x32x16_bf16 a[0:15], v[2:5], v[6:9], a[0:15]",
            "s_branch .LBB0_3",
            "v_accvgpr_read_b32 v30, a3",
            ".LBB0_3:",
            "s_nop 7", "s_nop 7", "s_nop 7", "s_nop 7",
            "v_accvgpr_read_b32 v31, a4"]
    assert not check(dead)
    # a VALU write reaching the product through a branch edge
    into = ["v_mov_b32 v4, 0", "s_cbranch_vccz .LBB0_5", "s_nop 7", ".LBB0_5:",
            "v_mfma_f32_32x32x16_bf16 v[10:25], v[2:5], v[6:9], 0"]
    assert check(into)


# ---- 2. VALU-written SGPR read by an LDS-DMA load ---------------------------

VALU_SGPR_TO_VMEM = 5
_SREG = re.compile(r"\bs\[(\d+):(\d+)\]|\bs(\d+)\b")


def _sregs(text: str) -> set[int]:
    out = set()
    for m in _SREG.finditer(text):
        if m.group(1):
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
        else:
            out.add(int(m.group(3)))
    return out


def sgpr_dma_hazards(lines: list[str]) -> list[str]:
    """Each global_load_lds whose SGPR operands a VALU instruction wrote fewer
    than VALU_SGPR_TO_VMEM wait states before, along any path into it."""
    instrs, succ = parse(lines)
    pred = _preds(succ)
    problems = []
    for i, (mn, ops) in enumerate(instrs):
        if not mn.startswith("global_load_lds"):
            continue
        need = _sregs(ops.split(",", 1)[1] if "," in ops else "")

        def back(j, ws):
            pm, pops = instrs[j]
            if _is_valu(pm) and _sregs(pops.split(",", 1)[0]) & need:
                problems.append(f"{pm} {pops} -> {mn} {ops} after {ws} wait states")
            return True
        back.cost = lambda j: _wait_states(*instrs[j])
        _walk(pred[i], pred, VALU_SGPR_TO_VMEM, back)
    return problems


@pytest.fixture(scope="module")
def all_kernel_asm(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    sys.path.insert(0, ROOT)
    from paged_kv_cache_58_amd import build as B
    out_dir = tmp_path_factory.mktemp("isa_all")
    procs = {}
    for src in B.SOURCES:
        if src in B.HOST_ONLY or not src.endswith(".hip"):
            continue
        out = out_dir / (src + ".s")
        cmd = [HIPCC, *B.DEVICE, *B.COMMON, *B.EXTRA.get(src, []), "-x", "hip", "-S",
               "--cuda-device-only", os.path.join(B.CSRC, src), "-o", str(out)]
        procs[src] = (subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE), out)
    asm = {}
    for src, (p, out) in procs.items():
        _, err = p.communicate()
        assert p.returncode == 0, err.decode()
        asm[src] = out.read_text()
    return asm


def test_lds_dma_sgpr_operands_settled(all_kernel_asm):
    assert any("global_load_lds_dwordx4" in a for a in all_kernel_asm.values())
    problems = []
    for src, text in all_kernel_asm.items():
        for body in _functions(text, "_Z"):
            problems += [f"{src}: {p}" for p in sgpr_dma_hazards(body)]
    assert not problems, "\n".join(problems[:20])


def test_sgpr_checker_catches_planted_hazard():
    bad = ["v_readlane_b32 s7, v248, 26", "s_mov_b32 m0, 0x25400",
           "global_load_lds_dword v0, s[6:7]"]
    assert sgpr_dma_hazards(bad)
    ok = ["v_readlane_b32 s7, v248, 26", "s_nop 4", "global_load_lds_dword v0, s[6:7]"]
    assert not sgpr_dma_hazards(ok)
    salu = ["s_add_u32 s6, s6, s8", "global_load_lds_dwordx4 v1, s[6:7] nt"]
    assert not sgpr_dma_hazards(salu)
    across = ["v_readlane_b32 s7, v248, 26", "s_cbranch_scc1 .LBB1_4", "s_nop 7", ".LBB1_4:",
              "global_load_lds_dword v0, s[6:7]"]
    assert sgpr_dma_hazards(across)


# 3. Serialized loads.  An empty asm that takes a just-loaded value as an
# operand makes the compiler wait for that load right there; with several
# such loads in a row (one per q fragment, say) every load then costs a full
# memory round trip before the next is issued.  Within a basic block, no
# kernel may issue three or more global loads that way, each waited for
# (vmcnt(0)) before the next one goes out.

def serialized_load_chains(lines: list[str], n: int = 3) -> list[int]:
    out, run, pending = [], 0, False
    for l in lines:
        t = l.split(";", 1)[0].strip()
        if t.startswith(".LBB") or t.startswith("s_cbranch") or t == "s_branch" or t.startswith("s_branch "):
            run, pending = 0, False
            continue
        if re.match(r"(global_load_dword|buffer_load_dword|flat_load_dword)", t):
            if pending:
                run = 0  # issued while another load was in flight: not serialized
            pending = True
        elif t.startswith("s_waitcnt") and "vmcnt(0)" in t and pending:
            run += 1
            pending = False
            if run >= n:
                out.append(run)
    return out


def test_no_serialized_load_chains(all_kernel_asm):
    problems = []
    for src, text in all_kernel_asm.items():
        for m in re.finditer(r"^(_Z\w+):", text, re.M):
            body = text[m.end():text.find(".Lfunc_end", m.end())].splitlines()
            if serialized_load_chains(body):
                problems.append(f"{src}: {m.group(1)}")
    assert not problems, "\n".join(problems[:20])


def test_chain_checker_catches_planted_chain():
    serial = []
    for k in range(4):
        serial += [f"global_load_dwordx4 v[{4 * k}:{4 * k + 3}], v[0:1], off offset:{64 * k}",
                   "s_waitcnt vmcnt(0)"]
    assert serialized_load_chains(serial)
    batched = [f"global_load_dwordx4 v[{4 * k}:{4 * k + 3}], v[0:1], off offset:{64 * k}"
               for k in range(4)] + ["s_waitcnt vmcnt(3)", "s_waitcnt vmcnt(0)"]
    assert not serialized_load_chains(batched)
    split = serial[:2] + [".LBB0_3:"] + serial[2:4] + ["s_cbranch_scc1 .LBB0_4"] + serial[4:]
    assert not serialized_load_chains(split)
