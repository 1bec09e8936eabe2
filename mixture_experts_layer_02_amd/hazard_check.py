"""Build-time check of the GEMM kernels' LDS-DMA wait states (gfx950 device assembly).

A buffer instruction that reads an SGPR needs five wait states after a VALU
instruction wrote that SGPR (readfirstlane, readlane - also as the reload of an
SGPR spilled to a VGPR lane -, compares and carry-outs with an SGPR result).
An LDS DMA also reads M0 (its LDS destination), so a VALU write of M0 counts.
Long branches (s_getpc / s_setpc) are followed to the labels they name.
The compiler cannot see that hazard through the inline-asm LDS DMA, so the
kernels insert the wait themselves: five states in general, one (for M0) in
the steady k-loop.  This script walks back from every `buffer_load_* ... lds`
of the generated code over all control-flow paths, counting wait states (one
per instruction, N+1 for s_nop N), and reports any VALU write of one of the
DMA's SGPR operands within five states.  build() fails on a report.

Usage: python hazard_check.py file.s [file.s ...]   (exit status 1 on a hazard)
"""
import re
import sys
from collections import defaultdict

# VALU instructions whose second operand is an SGPR result (carry-out / scale flag)
_SDST2 = re.compile(r"v_(add|sub|subrev|addc|subb|subbrev)_co_u32|v_div_scale_|v_mad_(u64_u32|i64_i32)")


def _sregs(tok):
    """SGPRs named by an operand token; M0 counts as the register "m0"."""
    tok = tok.strip().rstrip(",")
    if tok == "m0":
        return {"m0"}
    m = re.fullmatch(r"s\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.fullmatch(r"s(\d+)", tok)
    return {int(m.group(1))} if m else set()


def _functions(path):
    funcs, cur = [], None
    with open(path) as fh:
        for raw in fh:
            line = raw.split(";")[0].rstrip()
            s = line.strip()
            if not s:
                continue
            if re.match(r"^_Z\w+:$", line):
                cur = {"name": line[:-1], "insts": []}
                funcs.append(cur)
            elif cur is None:
                continue
            elif re.match(r"^\.L\w+:$", s):
                cur["insts"].append(("label", s[:-1]))
            elif not s.startswith("."):
                cur["insts"].append(("inst", s))
    return funcs


def check(path, out=sys.stdout):
    """(number of LDS-DMA instructions, number of hazards) in one assembly file."""
    total = bad = 0
    for f in _functions(path):
        ins = f["insts"]
        labels = {v: i for i, (k, v) in enumerate(ins) if k == "label"}
        preds = defaultdict(list)
        for i, (k, v) in enumerate(ins):
            if k != "inst":
                continue
            m = re.match(r"s_(cbranch_\w+|branch)\s+(\.L\w+)", v)
            if m and m.group(2) in labels:
                preds[labels[m.group(2)]].append(i)
            if re.match(r"s_setpc_b64\b", v):
                # A long branch: s_getpc, the target's offset added from a label
                # difference, s_setpc.  Its targets are the labels named since
                # the s_getpc; without one the jump is unknown and fails.
                targets = set()
                for j in range(i - 1, max(-1, i - 8), -1):
                    if ins[j][0] == "inst":
                        targets |= {t for t in re.findall(r"\.L\w+", ins[j][1]) if t in labels}
                        if re.match(r"s_getpc_b64\b", ins[j][1]):
                            break
                targets -= {t for t in targets if t.startswith(".Lpost_getpc")}
                if not targets:
                    bad += 1
                    print(f"unknown jump target in {f['name']}: {v!r}", file=out)
                for t in targets:
                    preds[labels[t]].append(i)
        for i, (k, v) in enumerate(ins):
            if k == "label":
                j = i - 1
                while j >= 0 and ins[j][0] == "label":
                    j -= 1
                if j >= 0 and not re.match(r"s_(branch|endpgm|setpc)\b", ins[j][1]):
                    preds[i].append(j)
        for i, (k, v) in enumerate(ins):
            if k != "inst" or not re.match(r"buffer_load_\w+\s", v) or not v.endswith(" lds"):
                continue
            total += 1
            need = {"m0"}  # the LDS destination base is read from M0
            for o in v.split(None, 1)[1].split(",")[1:]:
                for t in o.split():
                    need |= _sregs(t)
            stack, seen = [(i - 1, 0)], set()
            while stack:
                j, ws = stack.pop()
                if ws >= 5 or j < 0 or (j, ws) in seen:
                    continue
                seen.add((j, ws))
                kk, vv = ins[j]
                if kk == "label":
                    for p in preds.get(j, []):
                        stack.append((p, ws))
                    continue
                op = vv.split()[0]
                if op.startswith("v_") and " " in vv:
                    opnds = vv.split(None, 1)[1].split(",")
                    dst = _sregs(opnds[0].split()[0]) if opnds else set()
                    if _SDST2.match(op) and len(opnds) > 1:
                        dst |= _sregs(opnds[1].split()[0])
                    if dst & need:
                        bad += 1
                        print(f"hazard in {f['name']}: {vv!r} {ws} wait state(s) before {v!r}", file=out)
                m = re.match(r"s_nop\s+(\d+)", vv)
                stack.append((j - 1, ws + (int(m.group(1)) + 1 if m else 1)))
    return total, bad


if __name__ == "__main__":
    T = B = 0
    for p in sys.argv[1:]:
        t, b = check(p)
        T += t
        B += b
    print(f"{T} LDS-DMA instructions checked, {B} hazards")
    sys.exit(1 if B else 0)
