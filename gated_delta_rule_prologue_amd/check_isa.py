"""Build-time check of the scan and backward kernels' machine code (gfx950).

An MFMA whose accumulator input is the result of a recent MFMA, and whose
destination only partly overlaps that accumulator (the compiler allows the two
to be offset by two registers), produced corrupted results on MI355X when the
two products had different shapes (16x16x16 after 16x16x32 or the reverse):
their write-backs to the shared registers race.  Same-shape pairs laid out
this way are frequent in correct builds and are left alone.  Every kernel is
scanned for a mixed-shape pair; the build fails if one is found.

A DPP instruction reads its first source through the cross-lane network, which
needs two wait states after a VALU write of that register; the hardware does
not insert them.  The compiler does for its own DPP instructions, but not for
hand-written ones inside inline asm (the block inverse of the scan), so every
DPP instruction is checked against the two instructions before it.
"""
import re
import sys

_MFMA = re.compile(r"\s*(v_mfma_\S+)\s+([va])\[(\d+):(\d+)\],\s*[^,]+,\s*[^,]+,\s*([va])\[(\d+):(\d+)\]")
WINDOW = 24          # instructions after which an MFMA result is certainly written back


def scan(asm_text: str):
    bad = []
    recent = []      # (index, shape, kind, lo, hi) of recent MFMA destinations
    func = "?"
    n = 0
    for line in asm_text.splitlines():
        m = re.match(r"^(_Z\S+):", line)
        if m:
            func, recent, n = m.group(1), [], 0
            continue
        s = line.strip()
        if not s or s.startswith((";", ".")):
            continue
        n += 1
        mm = _MFMA.match(line)
        if not mm:
            continue
        shape = mm.group(1).split("_")[3]
        dk, d0, d1 = mm.group(2), int(mm.group(3)), int(mm.group(4))
        ck, c0, c1 = mm.group(5), int(mm.group(6)), int(mm.group(7))
        recent = [r for r in recent if n - r[0] <= WINDOW]
        mixed = any(k == ck and (lo, hi) == (c0, c1) and sh != shape
                    for (_, sh, k, lo, hi) in recent)
        partial = dk == ck and (d0, d1) != (c0, c1) and not (d1 < c0 or c1 < d0)
        if mixed and partial:
            bad.append((func, s))
        recent.append((n, shape, dk, d0, d1))
    return bad


_VR = re.compile(r"v\[(\d+):(\d+)\]")
_V1 = re.compile(r"v(\d+)$")


def _vgprs(op: str):
    op = op.strip().lstrip("-|")
    m = _VR.match(op)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = _V1.match(op)
    return {int(m.group(1))} if m else set()


def scan_dpp(asm_text: str):
    """DPP instructions whose first source was written by a VALU instruction
    fewer than two wait states before (s_nop N counts N + 1)."""
    bad = []
    hist = []        # (mnemonic, VGPRs written or s_nop count) of the last instructions
    func = "?"
    for line in asm_text.splitlines():
        m = re.match(r"^(_Z\S+):", line)
        if m:
            func, hist = m.group(1), []
            continue
        s = line.split(";")[0].strip()
        if not s or s.startswith(".") or s.endswith(":"):
            continue
        for ins in s.split("\n"):
            mnem, _, rest = ins.strip().partition(" ")
            ops = [o for o in rest.split(",")] if rest else []
            if "_dpp" in mnem and len(ops) >= 2:
                src = _vgprs(ops[1])
                ws = 0
                for pm, pw in reversed(hist):
                    if ws >= 2:
                        break
                    if pm == "s_nop":
                        ws += pw + 1
                        continue
                    if pm.startswith("v_") and pw & src:
                        bad.append((func, ins.strip()))
                        break
                    ws += 1
            if mnem == "s_nop":
                hist.append(("s_nop", int(ops[0], 0) if ops else 0))
            else:
                hist.append((mnem, _vgprs(ops[0]) if mnem.startswith("v_") and ops else set()))
            hist = hist[-8:]
    return bad


if __name__ == "__main__":
    text = open(sys.argv[1]).read()
    found = scan(text) + scan_dpp(text)
    for f, i in found:
        print(f[:80], i)
    print(len(found), "suspect instructions")
