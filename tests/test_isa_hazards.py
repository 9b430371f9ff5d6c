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
stops at labels and branches, so it covers each basic block on its own; the
kernel keeps every product chain and its fence inside one block.

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


def _instructions(asm: str, kernel_prefix: str) -> list[list[tuple[str, str]]]:
    """Basic blocks of every function whose name starts with kernel_prefix,
    as lists of (mnemonic, operand text)."""
    blocks: list[list[tuple[str, str]]] = []
    inside = False
    cur: list[tuple[str, str]] = []
    for line in asm.splitlines():
        if re.match(r"^_Z\w+:", line):
            inside = line.startswith(kernel_prefix)
            cur = []
            continue
        if not inside:
            continue
        s = line.split(";", 1)[0].strip()
        if not s:
            continue
        if s.endswith(":") or s.startswith("."):
            if cur:
                blocks.append(cur)
            cur = []
            if s.startswith(".Lfunc_end"):
                inside = False
            continue
        parts = s.split(None, 1)
        mn, ops = parts[0], parts[1] if len(parts) > 1 else ""
        cur.append((mn, ops))
        if mn.startswith("s_cbranch") or mn in ("s_branch", "s_endpgm", "s_setpc_b64"):
            blocks.append(cur)
            cur = []
    if cur:
        blocks.append(cur)
    return blocks


def _wait_states(mn: str, ops: str) -> int:
    if mn == "s_nop":
        return int(ops.strip(), 0) + 1
    return 1


def _is_valu(mn: str) -> bool:
    return mn.startswith("v_") and not mn.startswith("v_mfma")


def _dst(ops: str) -> set[tuple[str, int]]:
    first = ops.split(",", 1)[0]
    return _regs(first)


def check(blocks) -> list[str]:
    problems = []
    for blk in blocks:
        for i, (mn, ops) in enumerate(blk):
            if not mn.startswith("v_mfma"):
                continue
            fields = [f.strip() for f in ops.split(",")]
            dst, srcs = _regs(fields[0]), set()
            for f in fields[1:4]:
                srcs |= _regs(f)
            # VALU writes shortly before the product
            ws = 0
            for j in range(i - 1, -1, -1):
                pm, pops = blk[j]
                if ws >= VALU_TO_MFMA:
                    break
                if _is_valu(pm) and _dst(pops) & srcs:
                    problems.append(f"{pm} {pops} -> {mn} {ops} after {ws} wait states")
                ws += _wait_states(pm, pops)
            # uses of the result before it has drained
            ws = 0
            for j in range(i + 1, len(blk)):
                nm, nops = blk[j]
                if ws >= MFMA_DRAIN:
                    break
                if nm.startswith("v_mfma"):
                    nf = [f.strip() for f in nops.split(",")]
                    same_chain = _regs(nf[0]) == dst and _regs(nf[3]) == dst
                    touches = (_regs(nf[0]) | _regs(nf[1]) | _regs(nf[2]) | _regs(nf[3])) & dst
                    if touches and not same_chain:
                        problems.append(f"{mn} {ops} -> {nm} {nops} after {ws} wait states")
                    if same_chain:
                        break  # the chain's next link takes over the result
                elif _regs(nops) & dst:
                    problems.append(f"{mn} {ops} -> {nm} {nops} after {ws} wait states")
                ws += _wait_states(nm, nops)
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


def test_latent_kernel_has_products(latent_asm):
    blocks = _instructions(latent_asm, "_ZN2pa12_GLOBAL__N_123latent_partition_kernel")
    n = sum(1 for b in blocks for mn, _ in b if mn.startswith("v_mfma"))
    # three instantiations (1, 2 and 4 head tiles): per unit 36 / KS score
    # products (the wave's share of its tile's contraction, KS = 4 / tiles)
    # and 8 value products per head tile
    assert n >= (9 + 8) + (18 + 16) + (36 + 32)


def test_latent_kernel_mfma_hazards(latent_asm):
    blocks = _instructions(latent_asm, "_ZN2pa12_GLOBAL__N_123latent_partition_kernel")
    problems = check(blocks)
    assert not problems, "\n".join(problems[:20])


def test_checker_catches_planted_hazards():
    """The checker itself flags a VALU write right before a product and a
    read of a product's result before it drains, and passes a fenced chain."""
    bad = [[("v_mov_b32", "v4, 0"),
            ("v_mfma_f32_32x32x16_bf16", "v[10:25], v[2:5], v[6:9], 0")]]
    assert check(bad)
    bad2 = [[("v_mfma_f32_32x32x16_bf16", "v[10:25], v[2:5], v[6:9], 0"),
             ("v_add_f32_e32", "v30, v10, v11")]]
    assert check(bad2)
    ok = [[("v_mfma_f32_32x32x16_bf16", "v[10:25], v[2:5], v[6:9], 0"),
           ("ds_read_b128", "v[2:5], v40"),
           ("v_mfma_f32_32x32x16_bf16", "v[10:25], v[26:29], v[6:9], v[10:25]"),
           ("s_nop", "7"), ("s_nop", "7"), ("s_nop", "7"), ("s_nop", "7"),
           ("v_add_f32_e32", "v30, v10, v11")]]
    assert not check(ok)


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
    than VALU_SGPR_TO_VMEM wait states before (within its basic block)."""
    problems = []
    text = [l.split(";", 1)[0].strip() for l in lines]
    for i, l in enumerate(text):
        if not l.startswith("global_load_lds"):
            continue
        ops = l.split(None, 1)[1] if " " in l else ""
        need = _sregs(ops.split(",", 1)[1] if "," in ops else "")
        ws = 0
        for j in range(i - 1, -1, -1):
            p = text[j]
            if not p:
                continue
            if p.endswith(":") or p.startswith(".") or p.startswith("s_cbranch") or p == "s_branch":
                break
            if ws >= VALU_SGPR_TO_VMEM:
                break
            mn = p.split()[0]
            if _is_valu(mn) and " " in p and _sregs(p.split(None, 1)[1].split(",", 1)[0]) & need:
                problems.append(f"{p} -> {l} after {ws} wait states")
            ws += _wait_states(mn, p.split(None, 1)[1] if " " in p else "")
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
        problems += [f"{src}: {p}" for p in sgpr_dma_hazards(text.splitlines())]
    assert not problems, "\n".join(problems[:20])


def test_sgpr_checker_catches_planted_hazard():
    bad = ["v_readlane_b32 s7, v248, 26", "s_mov_b32 m0, 0x25400",
           "global_load_lds_dword v0, s[6:7]"]
    assert sgpr_dma_hazards(bad)
    ok = ["v_readlane_b32 s7, v248, 26", "s_nop 4", "global_load_lds_dword v0, s[6:7]"]
    assert not sgpr_dma_hazards(ok)
    salu = ["s_add_u32 s6, s6, s8", "global_load_lds_dwordx4 v1, s[6:7] nt"]
    assert not sgpr_dma_hazards(salu)


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
