"""Builds libmambascan.so (the HIP kernels and the C-ABI layer) for gfx950.

Run as ``python -m selective_state_space_27_amd.build`` or through
``__graft_entry__.build()``.  Each source is compiled to an object in
parallel, then linked into ``selective_state_space_27_amd/libmambascan.so``.

After compiling, the gfx950 code of each object is disassembled and checked
for one hazard the compiler cannot see: a DPP instruction written as inline
assembly (the scan's v_fmac_f32_dpp) must not read, as its lane-permuted
operand, a VGPR that a VALU instruction wrote less than two wait states
before (gfx9 family rule).  The build fails if one does.
"""
from __future__ import annotations

import concurrent.futures
import os
import re
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmambascan.so")
SOURCES = ["scan.hip", "scan_bwd.hip", "scan_bwd_wide.hip", "scan_fused_bwd.hip", "state_update.hip", "ssd.hip",
           "ssd_bwd.hip", "ssd_bwd_halves.hip", "mamba3.hip", "api.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed-fp32 instructions are kept out of the generated code (the compiler
# would otherwise form v_pk_{add,mul,fma}_f32 from scalar float code).
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-command-line-argument",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include")]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src + ".o")
    cmd = [HIPCC] + COMMON + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC] + COMMON + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (res.stderr or "").splitlines() if "is not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{errs}")
    return obj


LLVM = "/opt/rocm/llvm/bin"
# Sources whose kernels use inline-assembly DPP instructions.
DPP_CHECKED = ["scan.hip", "scan_bwd.hip"]
_VREG = re.compile(r"\bv(\d+)\b|\bv\[(\d+):(\d+)\]")


def _vregs(operand: str) -> set[int]:
    regs = set()
    for m in _VREG.finditer(operand):
        if m.group(1) is not None:
            regs.add(int(m.group(1)))
        else:
            regs.update(range(int(m.group(2)), int(m.group(3)) + 1))
    return regs


def _disassemble(obj: str) -> list[str]:
    """gfx950 disassembly of the device code bundled in a host object."""
    with tempfile.TemporaryDirectory() as tmp:
        fat, co = os.path.join(tmp, "fatbin"), os.path.join(tmp, "code.co")
        subprocess.run([f"{LLVM}/llvm-objcopy", f"--dump-section=.hip_fatbin={fat}", obj, os.path.join(tmp, "o")],
                       check=True, capture_output=True)
        subprocess.run([f"{LLVM}/clang-offload-bundler", "--type=o", f"--targets=hipv4-amdgcn-amd-amdhsa--{ARCH}",
                        f"--input={fat}", f"--output={co}", "--unbundle"], check=True, capture_output=True)
        out = subprocess.run([f"{LLVM}/llvm-objdump", "-d", f"--mcpu={ARCH}", co], check=True, capture_output=True,
                             text=True).stdout
    return out.splitlines()


def dpp_hazards(lines: list[str]) -> tuple[int, list[str]]:
    """(DPP instructions seen, violations): a DPP instruction whose first source
    (the lane-permuted one) a VALU instruction wrote within the two wait states
    before it, on any control-flow path into it (fall-through and every branch
    to a target in between are followed)."""
    insts = []  # (address, mnemonic, operands)
    for ln in lines:
        code = ln.split("//")[0].strip()
        m = re.search(r"//\s*([0-9A-Fa-f]+):", ln)
        if not code or code.endswith(":") or m is None:
            continue
        parts = code.split(None, 1)
        insts.append((int(m.group(1), 16), parts[0], parts[1] if len(parts) > 1 else ""))
    index = {a: i for i, (a, _, _) in enumerate(insts)}
    into = {}  # instruction index -> indices of branches that jump to it
    for i, (a, mnem, ops) in enumerate(insts):
        if mnem.startswith(("s_branch", "s_cbranch")):
            off = re.search(r"(-?\d+)\s*$", ops)
            if off is not None:  # signed 16-bit word offset from the next instruction (printed unsigned)
                o = int(off.group(1))
                o = o - 65536 if o >= 32768 else o
                t = index.get(a + 4 + 4 * o)
                if t is not None:
                    into.setdefault(t, []).append(i)

    def preds(i):
        out = list(into.get(i, []))
        if i > 0 and not insts[i - 1][1].startswith(("s_branch", "s_endpgm", "s_setpc")):
            out.append(i - 1)
        return out

    def writes(i):
        _, pm, pops = insts[i]
        if not pm.startswith("v_") or pm.startswith(("v_cmp", "v_readlane", "v_readfirstlane")):
            return set()
        pop = [o.strip() for o in pops.split(",")]
        dst = _vregs(pop[0]) if pop else set()
        if "swap" in pm and len(pop) > 1:
            dst |= _vregs(pop[1])
        return dst

    def cost(i):
        pm, pops = insts[i][1], insts[i][2]
        return int(pops.strip() or "0", 0) + 1 if pm.startswith("s_nop") else 1

    seen, bad = 0, []
    for i, (addr, mnem, ops) in enumerate(insts):
        if "_dpp" not in mnem or not mnem.startswith("v_"):
            continue
        seen += 1
        opnds = [o.strip() for o in ops.split(",")]
        src = _vregs(opnds[1]) if len(opnds) > 1 else set()
        stack = [(p, 0) for p in preds(i)]  # (instruction, wait states between it and the DPP instruction)
        while stack:
            j, w = stack.pop()
            if writes(j) & src:
                bad.append(f"{addr:#x} {mnem} {ops}: source written by {insts[j][1]} {insts[j][2]} "
                           f"{w} wait states before")
                break
            w += cost(j)
            if w < 2:
                stack.extend((p, w) for p in preds(j))
    return seen, bad


def check_dpp_hazards(verbose: bool = False) -> None:
    for src in DPP_CHECKED:
        seen, bad = dpp_hazards(_disassemble(os.path.join(BUILD, src + ".o")))
        if bad:
            raise RuntimeError(f"{src}: {len(bad)} DPP read-after-VALU-write hazards, e.g.\n" + "\n".join(bad[:10]))
        if verbose:
            print(f"{src}: {seen} DPP instructions, no read-after-VALU-write hazard")


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    check_dpp_hazards(verbose)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
