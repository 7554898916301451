"""Wait-state check of the hand-written inline asm in the gfx950 assembly of the product sources.

The compiler inserts the wait states that CDNA hazards need between instructions it can see, but
not around instructions inside inline asm: it does not know what they read or write. The LLVM
assembly printer brackets every inline-asm block with `;;#ASMSTART` / `;;#ASMEND`, so the
instructions the asm contributed can be checked against the hazard entries they rely on, on
every path through the compiled code (branches followed in both directions):

  D1  a VALU write of an SGPR, then a vector-memory instruction that reads it (the LDS DMA's
      64-bit base address): 5 wait states;
  D2  a VALU write of M0, then the LDS DMA that takes its LDS address from M0: 5 wait states
      (as D1); an SALU write of M0 before it: 1 wait state;
  M1  a VALU write of a VGPR or AGPR, then an MFMA that reads it as an operand: 2 wait states;
  M2  an MFMA writing AGPRs, then any other instruction reading or writing them: 18 wait states
      (the largest MFMA figure; the 32x32x16 bf16 MFMA has 8 passes and needs fewer), except a
      following MFMA that accumulates into exactly the same registers (no wait).

A wait state is one issued instruction; `s_nop N` supplies N + 1. Counting every other
instruction as one is the conservative reading.
"""
import re

_REG = re.compile(r"^([vsa])\[(\d+):(\d+)\]$|^([vsa])(\d+)$")
_SPECIAL = {"vcc": {("s", "vcc_lo"), ("s", "vcc_hi")}, "vcc_lo": {("s", "vcc_lo")}, "vcc_hi": {("s", "vcc_hi")},
            "m0": {("m0", 0)}, "exec": {("s", "exec_lo"), ("s", "exec_hi")}}


def regs(tok):
    """Registers named by one operand token: a set of (file, index)."""
    tok = tok.strip().rstrip(",")
    if tok in _SPECIAL:
        return set(_SPECIAL[tok])
    m = _REG.match(tok)
    if not m:
        return set()
    if m.group(1):
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    return {(m.group(4), int(m.group(5)))}


class Insn:
    def __init__(self, text, asm, line):
        self.text, self.asm, self.line = text, asm, line
        parts = text.split(None, 1)
        self.op = parts[0]
        self.args = [a.strip() for a in parts[1].split(",")] if len(parts) > 1 else []
        self.label = None
        self.target = None
        if self.op.startswith(("s_branch", "s_cbranch")) and self.args:
            self.target = self.args[0]

    def waits(self):
        if self.op == "s_nop":
            return int(self.args[0], 0) + 1
        return 1

    def is_valu(self):
        return self.op.startswith("v_")

    def is_mfma(self):
        return self.op.startswith("v_mfma")

    def defs(self):
        a = self.args
        if not a:
            return set()
        if self.is_valu():
            if self.op.startswith(("v_cmpx",)):
                return set(_SPECIAL["exec"])
            if self.op.startswith(("v_readfirstlane", "v_readlane", "v_cmp")):
                return regs(a[0])
            if "_co_" in self.op or self.op.startswith("v_div_scale"):
                return regs(a[0]) | (regs(a[1]) if len(a) > 1 else set())
            return regs(a[0])
        if self.op.startswith("s_") and not self.op.startswith(("s_nop", "s_waitcnt", "s_cbranch", "s_branch",
                                                                  "s_barrier", "s_setprio", "s_endpgm")):
            return regs(a[0])
        return set()

    def uses(self):
        a = self.args
        if self.is_valu() and len(a) > 1:
            start = 2 if ("_co_" in self.op or self.op.startswith("v_div_scale")) else 1
            out = set()
            for t in a[start:]:
                out |= regs(t)
            return out
        out = set()
        for t in a:
            out |= regs(t)
        return out


def parse(text):
    """Functions of an assembly file: name -> list of Insn and local-label names (str)."""
    funcs, cur, in_asm = {}, None, False
    for n, raw in enumerate(text.splitlines(), 1):
        s = raw.strip()
        if s.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if s.startswith(";;#ASMEND"):
            in_asm = False
            continue
        line = s.split(";")[0].strip()
        if not line:
            continue
        if line.endswith(":"):
            name = line[:-1]
            if name.startswith((".L", "$")):
                if cur is not None:
                    cur.append(name)
            else:
                cur = funcs.setdefault(name, [])
            continue
        if line.startswith(".") or cur is None:
            continue
        cur.append(Insn(line, in_asm, n))
    return funcs


class Flow:
    """Predecessors and successors over one function's instruction list (labels are nodes too)."""

    def __init__(self, body):
        self.body = body
        self.label_at = {x: i for i, x in enumerate(body) if isinstance(x, str)}
        self.preds = {i: [] for i in range(len(body))}
        for i, x in enumerate(body):
            for j in self.succ(i):
                self.preds[j].append(i)

    def succ(self, i):
        x = self.body[i]
        out = []
        if isinstance(x, Insn):
            if x.target is not None and x.target in self.label_at:
                out.append(self.label_at[x.target])
            if x.op.startswith(("s_branch", "s_endpgm", "s_setpc", "s_trap")):
                return out
        if i + 1 < len(self.body):
            out.append(i + 1)
        return out


def _search(flow, start, budget, step, hit):
    """Visit instructions reachable from `start` (exclusive) in direction `step` (flow.succ or
    flow.preds) while fewer than `budget` wait states have passed; hit(insn, waits_before) returns
    a message for a violation. Returns the messages found."""
    found, best = [], {}
    stack = [(j, 0) for j in step(start)]
    while stack:
        i, w = stack.pop()
        if w >= budget or best.get(i, budget + 1) <= w:
            continue
        best[i] = w
        x = flow.body[i]
        if isinstance(x, Insn):
            msg = hit(x, w)
            if msg:
                found.append(msg)
                continue
            w2 = w + x.waits()
        else:
            w2 = w
        stack.extend((j, w2) for j in step(i))
    return found


def check_function(name, body):
    """Violations of D1, D2, M1, M2 by the inline-asm instructions of one function."""
    flow = Flow(body)
    back = lambda i: flow.preds[i]
    fwd = flow.succ
    out = []
    for i, x in enumerate(body):
        if not isinstance(x, Insn) or not x.asm:
            continue
        where = f"{name} line {x.line}: {x.text}"
        if x.op.startswith("global_load_lds"):
            base = regs(x.args[1]) if len(x.args) > 1 else set()
            m0 = set(_SPECIAL["m0"])

            def d1(y, w, base=base, m0=m0):
                if y.is_valu() and (y.defs() & (base | m0)):
                    return f"D1/D2: {where} reads a register written by `{y.text}` {w} wait states before"
                if not y.is_valu() and w < 1 and (y.defs() & m0):
                    return f"D2: {where} reads M0 written by `{y.text}` with no wait state"
                return None
            out += _search(flow, i, 5, back, d1)
        elif x.is_mfma():
            srcs = set()
            for t in x.args[1:]:
                srcs |= regs(t)

            def m1(y, w, srcs=srcs):
                if y.is_valu() and not y.is_mfma() and (y.defs() & srcs):
                    return f"M1: {where} reads a register written by `{y.text}` {w} wait states before"
                return None
            out += _search(flow, i, 2, back, m1)
            dst = regs(x.args[0])
            if any(f == "a" for f, _ in dst):
                def m2(y, w, dst=dst, x=x):
                    if y.is_mfma():
                        if regs(y.args[0]) == dst and len(y.args) > 3 and regs(y.args[3]) == dst:
                            return None          # accumulation into the same registers
                        touched = set()
                        for t in y.args:
                            touched |= regs(t)
                        if touched & dst:
                            return f"M2: `{y.text}` touches {where}'s result {w} wait states after it"
                        return None
                    if (y.uses() | y.defs()) & dst:
                        return f"M2: `{y.text}` touches {where}'s result {w} wait states after it"
                    return None
                out += _search(flow, i, 18, fwd, m2)
    return out


def check(text):
    """All violations in an assembly file, and the number of inline-asm DMA and MFMA sites seen."""
    found, sites = [], 0
    for name, body in parse(text).items():
        sites += sum(1 for x in body if isinstance(x, Insn) and x.asm and
                     (x.op.startswith("global_load_lds") or x.is_mfma()))
        found += check_function(name, body)
    return found, sites
