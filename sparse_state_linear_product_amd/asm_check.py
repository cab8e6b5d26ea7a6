"""Build-time check of the kernels' inline-assembly loads.

The kernels that stage memory through LDS with LDS-DMA (the chunk-parallel
SDM kernels, the GDN state kernel) read that LDS with inline-assembly loads
(ds_read_*, waited for by an explicit `s_waitcnt lgkmcnt(0)`), and the SDM
chunked backward prefetches with inline-assembly global loads
(global_load_dwordx4, waited for by an explicit `s_waitcnt vmcnt(0)`), so
that the compiler cannot move them or wait for the DMAs in flight before
them.  The compiler treats the destination
registers of such a load as written when the asm statement ends, so nothing
in the language stops the register allocator from copying, spilling or
reusing them before the data has arrived.  This check reads the generated
gfx950 assembly and fails if any instruction outside inline assembly touches
a destination register of such a load before a wait that covers it, along any
path of the control-flow graph (a forward dataflow over basic blocks, to a
fixpoint across loop back-edges).
"""
import os
import re
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CHECKED = ["sdm_chunk.hip", "sdm_chunk_bwd.hip", "gdn_chunk.hip"]

_VREG = re.compile(r"\b([va])(\d+)\b|\b([va])\[(\d+):(\d+)\]")
_LABEL = re.compile(r"^(\.?L?BB[\w.]+|\.LBB[\w.]+):")
# a basic block that no branch targets carries its label only as a comment
_FALL_LABEL = re.compile(r"^;\s*(%bb\.\d+):")
_BRANCH = re.compile(r"^\s*(s_branch|s_cbranch_\w+)\s+(\S+)")


def _regs(text):
    out = set()
    for m in _VREG.finditer(text):
        if m.group(1):
            out.add((m.group(1), int(m.group(2))))
        else:
            for r in range(int(m.group(4)), int(m.group(5)) + 1):
                out.add((m.group(3), r))
    return out


def _kernel_bodies(asm):
    """(name, lines) of every kernel in a device assembly file."""
    bodies, cur, name = [], None, None
    for line in asm.splitlines():
        m = re.match(r"^(_Z\w+):", line)
        if m:
            name, cur = m.group(1), []
            continue
        if cur is not None:
            cur.append(line)
            if "s_endpgm" in line:
                bodies.append((name, cur))
                cur = None
    return bodies


def _blocks(lines):
    """Basic blocks as (label, [items], successors); items are ('asm', text) for
    an inline-asm region, ('ins', text) for a compiler instruction."""
    blocks, cur, label, in_asm, asm_buf = [], [], "entry", False, []
    for raw in lines:
        line = raw.split(";")[0].rstrip() if not raw.strip().startswith(";;#ASM") else raw.strip()
        if raw.strip() == ";;#ASMSTART":
            in_asm, asm_buf = True, []
            continue
        if raw.strip() == ";;#ASMEND":
            in_asm = False
            cur.append(("asm", "\n".join(asm_buf)))
            continue
        if in_asm:
            asm_buf.append(raw.strip())
            continue
        m = _LABEL.match(raw.strip()) or _FALL_LABEL.match(raw.strip())
        if m:
            blocks.append([label, cur, None])
            label, cur = m.group(1), []
            continue
        if not line.strip() or line.strip().startswith("."):
            continue
        cur.append(("ins", line.strip()))
    blocks.append([label, cur, None])
    # successors: explicit branch targets, plus fallthrough unless an
    # unconditional branch or the end of the program ends the block
    for i, blk in enumerate(blocks):
        succ = []
        fall = True
        for kind, text in blk[1]:
            if kind != "ins":
                continue
            b = _BRANCH.match(text)
            if b:
                succ.append(b.group(2))
                if b.group(1) == "s_branch":
                    fall = False
            if text.startswith("s_endpgm"):
                fall = False
        if fall and i + 1 < len(blocks):
            succ.append(blocks[i + 1][0])
        blk[2] = succ
    return blocks


def _transfer(items, pending, report):
    """pending: frozenset of (reg, counter); returns the set after the block."""
    pend = set(pending)
    for kind, text in items:
        if kind == "asm":
            for ln in text.splitlines():
                op = ln.split()[0] if ln.split() else ""
                if op.startswith("s_waitcnt"):
                    if "vmcnt(0)" in ln:
                        pend = {p for p in pend if p[1] != "vm"}
                    if "lgkmcnt(0)" in ln:
                        pend = {p for p in pend if p[1] != "lgkm"}
                elif op.startswith("global_load") or op.startswith("ds_read"):
                    dst = ln.split(None, 1)[1].split(",")[0]
                    cnt = "vm" if op.startswith("global_load") else "lgkm"
                    for r in _regs(dst):
                        pend.add((r, cnt))
            continue
        op = text.split()[0]
        if op.startswith("s_waitcnt"):
            if "vmcnt(0)" in text:
                pend = {p for p in pend if p[1] != "vm"}
            if "lgkmcnt(0)" in text:
                pend = {p for p in pend if p[1] != "lgkm"}
            continue
        touched = _regs(text)
        bad = {p for p in pend if p[0] in touched}
        if bad and report is not None:
            report.append((text, sorted(p[0] for p in bad)))
    return frozenset(pend)


def count_asm_loads(lines):
    """Number of inline-asm global/LDS loads in a kernel body."""
    n, in_asm = 0, False
    for raw in lines:
        t = raw.strip()
        if t == ";;#ASMSTART":
            in_asm = True
        elif t == ";;#ASMEND":
            in_asm = False
        elif in_asm and (t.startswith("global_load") or t.startswith("ds_read")):
            n += 1
    return n


def check_kernel(lines):
    """Instructions that touch an inline-asm load's destination before its wait."""
    blocks = _blocks(lines)
    index = {b[0]: i for i, b in enumerate(blocks)}
    pin = {b[0]: frozenset() for b in blocks}
    work = [b[0] for b in blocks]
    while work:
        lab = work.pop(0)
        blk = blocks[index[lab]]
        out = _transfer(blk[1], pin[lab], None)
        for s in blk[2]:
            if s in pin and not out <= pin[s]:
                pin[s] = pin[s] | out
                work.append(s)
    report = []
    for blk in blocks:
        _transfer(blk[1], pin[blk[0]], report)
    return report


def run(verbose=False):
    """Compile the checked sources to gfx950 assembly and verify them; raises on a violation."""
    flags = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Xclang", "-target-feature",
             "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "--cuda-device-only",
             "-S"]
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    problems, counts = [], {}
    with tempfile.TemporaryDirectory() as tmp:
        for name in CHECKED:
            out = os.path.join(tmp, name + ".s")
            subprocess.run([hipcc] + flags + [os.path.join(HERE, "csrc", name), "-o", out],
                           check=True, capture_output=True)
            asm = open(out).read()
            counts[name] = 0
            for kname, lines in _kernel_bodies(asm):
                counts[name] += count_asm_loads(lines)
                for text, regs in check_kernel(lines):
                    problems.append(f"{name}:{kname}: '{text}' touches {regs} before the wait")
            if verbose:
                print(f"asm_check: {name}: {counts[name]} inline-asm loads, every destination "
                      f"untouched until its wait", flush=True)
    if problems:
        raise RuntimeError("inline-asm load registers used before their wait:\n" +
                           "\n".join(problems[:20]))
    return counts


if __name__ == "__main__":
    run(verbose=True)
    sys.exit(0)
