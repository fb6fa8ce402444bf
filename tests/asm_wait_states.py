"""Wait states around inline assembly in compiled gfx950 code.

gfx950 requires independent instructions between some dependent pairs: a
VALU result read by a matrix instruction (2 wait states), a VALU result
read by a DPP or row-swap permute (2), a transcendental result read by the
next VALU instruction (1), a matrix result read by a VALU instruction
(several).  The compiler inserts them only around instructions it
generates; instructions written in inline asm are outside that check.  This
module scans the assembly text of a build for such pairs in which one side
is inline asm (straight-line code; a label is crossed backwards unless the
instruction before it is an unconditional branch or the end of the
program)."""
import re

TRANS = ("v_exp_f32", "v_log_f32", "v_rcp_f32", "v_rsq_f32", "v_sqrt_f32", "v_sin_f32", "v_cos_f32",
         "v_exp_f16", "v_rcp_f16", "v_sqrt_f16", "v_rsq_f16", "v_log_f16", "v_rcp_iflag_f32")
MFMA_TO_VALU = 19   # conservative bound for the longest matrix instructions


def parse(text):
    """[(line, instruction, inside_inline_asm)], with 'LABEL' entries."""
    out, inasm = [], False
    for i, line in enumerate(text.split("\n")):
        s = line.strip()
        if s.startswith(";;#ASMSTART"):
            inasm = True
            continue
        if s.startswith(";;#ASMEND"):
            inasm = False
            continue
        s = s.split(";")[0].strip()
        if re.match(r"^(\.LBB\S*|[_A-Za-z]\S*):", s):
            out.append((i, "LABEL", False))
            continue
        if not line.startswith("\t") or not s or s.startswith("."):
            continue
        out.append((i, s, inasm))
    return out


def _regs(tok):
    r = set()
    for m in re.finditer(r"v\[(\d+):(\d+)\]|\bv(\d+)\b", tok):
        if m.group(3):
            r.add(int(m.group(3)))
        else:
            r.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return r


def _ops(s):
    return [o.strip() for o in s.split(" ", 1)[1].split(",")] if " " in s else []


def _dst(s):
    o = _ops(s)
    if not o or not s.startswith("v_") or s.startswith(("v_cmp", "v_readlane", "v_readfirstlane")):
        return set()
    return _regs(o[0])


def _srcs(s):
    o, r = _ops(s), set()
    for x in o[1:]:
        r |= _regs(x)
    if s.startswith("v_permlane") and o:
        r |= _regs(o[0])
    return r


def _wait_states(s):
    m = re.match(r"s_nop\s+(\w+)", s)
    return int(m.group(1), 0) + 1 if m else 1


def _back(inst, k, limit):
    w, j = 0, k - 1
    while j >= 0 and w < limit:
        s = inst[j][1]
        if s == "LABEL":
            if j > 0 and inst[j - 1][1].split()[0] in ("s_branch", "s_endpgm", "s_setpc_b64"):
                return
            j -= 1
            continue
        yield inst[j], w
        w += _wait_states(s)
        j -= 1


def violations(text):
    """[(kind, line, consumer, producer, wait_states)] in one assembly file."""
    inst, found = parse(text), []
    for k, (i, s, a) in enumerate(inst):
        if s == "LABEL":
            continue
        mn = s.split()[0]
        perm = mn.startswith("v_permlane") or "dpp" in mn or re.search(r"\b(row_|quad_perm|row_bcast)", s)
        if mn.startswith("v_mfma") or perm:
            live = set()
            if mn.startswith("v_mfma"):
                for x in _ops(s)[1:4]:
                    live |= _regs(x)
            else:
                live = _srcs(s)
            for (pi, ps, pa), w in _back(inst, k, 2):
                d = _dst(ps)
                if pa and ps.startswith("v_") and d & live:
                    found.append(("asm VALU -> " + ("MFMA" if mn.startswith("v_mfma") else "permute"), i, s, ps, w))
                live -= d
                if not live:
                    break
        if a and s.startswith("v_"):
            live = _srcs(s)
            for (pi, ps, pa), w in _back(inst, k, MFMA_TO_VALU):
                d = _dst(ps)
                if d & live:
                    pm = ps.split()[0]
                    if pm.startswith(TRANS) and w < 1:
                        found.append(("transcendental -> asm VALU", i, s, ps, w))
                    if pm.startswith("v_mfma"):
                        found.append(("MFMA -> asm VALU", i, s, ps, w))
                live -= d
                if not live:
                    break
    return found
