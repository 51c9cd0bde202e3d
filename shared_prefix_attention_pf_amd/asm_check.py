"""Wait-state check of the generated gfx950 assembly of the bf16 kernels.

The accumulating products of the bf16 kernels are inline-asm MFMAs writing
AGPRs.  The compiler inserts wait states for the MFMAs it generates itself,
but it does not know an asm statement's latency, so any instruction it places
after an asm product that touches that product's destination registers (a copy
between register files, a spill, a VALU read) could see the old value.  This
check scans the assembly and reports every instruction, other than another
asm product accumulating into exactly the same registers, that names a
destination register of an asm product within `WAIT_STATES` wait states of it.

    python shared_prefix_attention_pf_amd/asm_check.py file.s

Exit status 1 when a violation is found.
"""
import re
import sys

# XDL write -> VALU/memory access of the result: 8-pass products need 11 wait
# states on gfx940-class hardware; allow margin for gfx950's extra pass.
WAIT_STATES = 12
# the same for 16-pass products (v_mfma_f32_32x32x2_f32): 19, with margin
WAIT_STATES_16PASS = 20

_AREG = re.compile(r"\ba(\d+)\b|\ba\[(\d+):(\d+)\]")
_MFMA_DST = re.compile(r"^\s*v_mfma\w*\s+a\[(\d+):(\d+)\],\s*(\S+),\s*(\S+),\s*a\[(\d+):(\d+)\]")


def _aregs(text):
    out = set()
    for m in _AREG.finditer(text):
        if m.group(1) is not None:
            out.add(int(m.group(1)))
        else:
            out.update(range(int(m.group(2)), int(m.group(3)) + 1))
    return out


def _wait_states(line):
    s = line.strip()
    m = re.match(r"s_nop\s+(\d+)", s)
    if m:
        return int(m.group(1)) + 1
    if not s or s.startswith(";") or s.startswith(".") or s.endswith(":"):
        return 0
    return 1


def check(lines, wait_states=WAIT_STATES):
    """Returns a list of (line number, message) violations; `wait_states` is
    the distance an asm product's destination must be left alone (12 for the
    8-pass bf16 products, more for the 16-pass fp32 ones)."""
    bad = []
    in_asm = False
    pending = []   # [dst register set, remaining wait states, line number]
    for no, raw in enumerate(lines, 1):
        line = raw.split(";;")[0] if "ASM" not in raw else raw
        s = line.strip()
        if s.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if s.startswith(";;#ASMEND"):
            in_asm = False
            continue
        code = s.split(";")[0].strip()
        if not code or code.endswith(":") or code.startswith("."):
            continue
        mf = _MFMA_DST.match(code)
        if in_asm and mf:
            dst = set(range(int(mf.group(1)), int(mf.group(2)) + 1))
            src_c = set(range(int(mf.group(5)), int(mf.group(6)) + 1))
            srcs_ab = _aregs(mf.group(3)) | _aregs(mf.group(4))
            for regs, _left, at in pending:
                if regs & srcs_ab:
                    bad.append((no, f"asm MFMA reads a product of line {at} as A/B operand"))
                if regs & (dst | src_c) and not (regs == dst and dst == src_c):
                    bad.append((no, f"asm MFMA partially overlaps the product of line {at}"))
            pending = [p for p in pending if not (p[0] == dst)]
            pending.append([dst, wait_states, no])
            # the product's own issue does not count toward later wait states
            continue
        used = _aregs(code)
        for regs, _left, at in pending:
            if regs & used:
                bad.append((no, f"'{code}' touches the destination of the asm MFMA at line {at} "
                                f"within {wait_states} wait states"))
        ws = _wait_states(code)
        for p in pending:
            p[1] -= ws
        pending = [p for p in pending if p[1] > 0]
        if code.startswith("s_branch") or code.startswith("s_cbranch") or code.startswith("s_setpc"):
            # control flow: the successor may be anywhere; stay conservative by
            # keeping the pending products (they are checked in fall-through
            # order, which is how the blocks are laid out)
            pass
    return bad


def check_m0(lines):
    """M0 is set by the inline-asm staging loads right before they use it;
    any other instruction touching M0 could see or clobber that value."""
    bad = []
    in_asm = False
    for no, raw in enumerate(lines, 1):
        st = raw.strip()
        if st.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if st.startswith(";;#ASMEND"):
            in_asm = False
            continue
        code = st.split(";")[0]
        if not in_asm and re.search(r"\bm0\b", code):
            bad.append((no, f"'{code.strip()}' uses M0 outside an inline-asm staging load"))
    return bad


def check_no_stack(lines):
    """Kernels must keep everything in registers: a private segment means an
    array was placed in scratch memory (a slow path inside the loops)."""
    bad = []
    for no, raw in enumerate(lines, 1):
        m = re.match(r"\s*\.private_segment_fixed_size:\s+(\d+)", raw)
        if m and int(m.group(1)) != 0:
            bad.append((no, f"kernel uses {m.group(1)} bytes of scratch memory"))
    return bad


def main(argv):
    if len(argv) != 2:
        print(__doc__)
        return 2
    with open(argv[1]) as fh:
        lines = fh.readlines()
    bad = check(lines) + check_no_stack(lines) + check_m0(lines)
    for no, msg in bad[:50]:
        print(f"{argv[1]}:{no}: {msg}")
    if bad:
        print(f"{len(bad)} wait-state violation(s)")
        return 1
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))
