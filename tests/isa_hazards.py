"""Software wait-state checks on gfx950 device assembly produced from this
repository's kernels (``hipcc --cuda-device-only -S``).

CDNA3/CDNA4 hardware does not interlock a few register dependencies of the
matrix (XDL) pipeline and of M0: the program must place independent
instructions or ``s_nop`` between producer and consumer.  The compiler's
hazard recognizer does this for the instructions it knows, but an inline
assembly statement is opaque to it, so the emitted code is checked here.

The required minimum for each pattern is read from the compiler itself:
``tests/isa/probe.hip`` holds one small kernel per pattern, and the wait
states its hazard recognizer leaves there (the tightest producer/consumer
pair of that kind) become the bound.  Patterns (wait states = instructions
issued in between, ``s_nop N`` counting N + 1):

* an XDL op writes registers that a later non-XDL instruction reads or
  writes, or that a later XDL op reads as SrcA/SrcB or as a SrcC that is
  not exactly those registers (``raw``); a later XDL op whose SrcC is
  exactly those registers (accumulation, ``srcc``) has its own bound;
* a VALU instruction (v_accvgpr_* included) writes a register that an XDL
  op then reads (``valu_xdl``);
* an SALU instruction writes M0 that an LDS-DMA load (``... lds``) then
  reads (``m0_dma``);
* a VALU instruction writes a scalar register (v_readfirstlane, a compare,
  a carry out) that a vector memory instruction then reads as its
  descriptor, offset or address (``valu_sgpr_vmem``; counted from the last
  VALU write even if a scalar instruction rewrote the register since, as
  the compiler does).

Two XDL ops writing the same registers, and an XDL op's SrcC overwritten
by a later instruction, are left to the compiler: the library names no
XDL op in inline assembly (checked from the sources), so the hazard
recognizer sees every one of them.  Paths follow fall-through and branch
targets, loop back-edges included.
"""
import re
from dataclasses import dataclass, field

MAX_WINDOW = 24          # no bound checked here exceeds this many wait states

_REG = re.compile(r"^([vas])(?:(\d+)|\[(\d+):(\d+)\])$")


def _regs(op):
    """Registers of one operand as a set of ('v'|'a'|'s', index); vcc is
    s106:s107 on this target."""
    op = op.strip()
    if op in ("vcc", "vcc_lo", "vcc_hi"):
        return {("s", 106), ("s", 107)} if op == "vcc" else {("s", 106 if op == "vcc_lo" else 107)}
    m = _REG.match(op)
    if not m:
        return set()
    kind = m.group(1)
    if m.group(2) is not None:
        return {(kind, int(m.group(2)))}
    return {(kind, i) for i in range(int(m.group(3)), int(m.group(4)) + 1)}


@dataclass
class Inst:
    text: str
    op: str
    operands: list
    defs: set = field(default_factory=set)
    uses: set = field(default_factory=set)
    srcc: set = field(default_factory=set)
    srcab: set = field(default_factory=set)
    branch: str = None          # target label
    cond: bool = False
    writes_m0: bool = False
    reads_m0_dma: bool = False

    @property
    def is_xdl(self):
        return self.op.startswith("v_mfma")

    @property
    def is_valu(self):
        return self.op.startswith("v_") and not self.is_xdl

    @property
    def is_vmem(self):
        return self.op.startswith(("buffer_", "global_", "flat_", "scratch_"))

    @property
    def vdefs(self):
        return {r for r in self.defs if r[0] != "s"}

    @property
    def sdefs(self):
        return {r for r in self.defs if r[0] == "s"}

    @property
    def wait_states(self):
        if self.op == "s_nop":
            return int(self.operands[0], 0) + 1
        return 1


def _split_operands(rest):
    out, depth, cur = [], 0, ""
    for ch in rest:
        if ch == "[":
            depth += 1
        elif ch == "]":
            depth -= 1
        if ch == "," and depth == 0:
            out.append(cur.strip())
            cur = ""
        else:
            cur += ch
    if cur.strip():
        out.append(cur.strip())
    return out


def parse_inst(line):
    parts = line.split(None, 1)
    op = parts[0]
    rest = parts[1] if len(parts) > 1 else ""
    # modifiers after the operands (offen, lds, offset:..., glc) are words
    # without commas; keep only comma-separated operand fields
    ops = _split_operands(rest)
    if ops:
        tail = ops[-1].split()
        ops[-1] = tail[0] if tail else ""
        mods = tail[1:]
    else:
        mods = []
    ins = Inst(line, op, ops)
    regs = [_regs(o) for o in ops]
    if ins.is_xdl:
        ins.defs = regs[0]
        ins.srcab = regs[1] | regs[2]
        ins.srcc = regs[3]
        ins.uses = ins.srcab | ins.srcc
    elif op.startswith("v_"):
        # results: the first operand, plus the scalar carry/condition output
        # of the two-result forms
        n_out = 2 if op.startswith(("v_add_co", "v_sub_co", "v_subrev_co", "v_addc_co",
                                    "v_subb_co", "v_subbrev_co", "v_mad_u64", "v_mad_i64",
                                    "v_div_scale")) and len(regs) > 2 else 1
        if op.startswith("v_cmpx"):
            n_out = 0                      # writes EXEC only
        ins.defs = set().union(*regs[:n_out]) if regs and n_out else set()
        ins.uses = set().union(*regs[n_out:]) if len(regs) > n_out else set()
        if op.endswith("_e32") and op.startswith(("v_cndmask", "v_addc_co", "v_subb_co",
                                                  "v_subbrev_co")):
            ins.uses |= {("s", 106), ("s", 107)}
    elif op.startswith("ds_"):
        if op.startswith(("ds_write", "ds_store")) or op in ("ds_nop",):
            ins.uses = set().union(*regs) if regs else set()
        else:
            ins.defs = regs[0] if regs else set()
            ins.uses = set().union(*regs[1:]) if len(regs) > 1 else set()
    elif op.startswith(("buffer_", "global_", "flat_", "scratch_")):
        is_load = "_load" in op or "_atomic" in op
        dma = "lds" in mods or op.endswith("_lds") or "_lds_" in op
        if dma:
            ins.uses = set().union(*regs) if regs else set()
            ins.reads_m0_dma = True
        elif is_load:
            ins.defs = regs[0] if regs else set()
            ins.uses = set().union(*regs[1:]) if len(regs) > 1 else set()
        else:
            ins.uses = set().union(*regs) if regs else set()
    elif op.startswith("s_"):
        if ops and ops[0] == "m0" and not op.startswith(("s_cmp", "s_bitcmp", "s_cbranch")):
            ins.writes_m0 = True
        if op == "s_branch" or op.startswith("s_cbranch"):
            ins.branch = ops[0]
            ins.cond = op.startswith("s_cbranch")
    return ins


def split_functions(asm_text):
    """{symbol: [Inst]} and {symbol: {label: index}} for every kernel body."""
    funcs, labels = {}, {}
    cur = None
    for raw in asm_text.splitlines():
        line = raw.split(";", 1)[0].rstrip()
        if not line.strip():
            continue
        s = line.strip()
        if not raw.startswith((" ", "\t")) and s.endswith(":") and not s.startswith("."):
            cur = s[:-1]
            funcs[cur], labels[cur] = [], {}
            continue
        if cur is None:
            continue
        if s.startswith(".Lfunc_end"):
            cur = None
            continue
        if s.endswith(":"):
            labels[cur][s[:-1]] = len(funcs[cur])
            continue
        if s.startswith("."):
            continue
        funcs[cur].append(parse_inst(s))
    return funcs, labels


def _successors(insts, labels, j):
    ins = insts[j]
    if ins.op in ("s_endpgm", "s_setpc_b64"):
        return []
    if ins.branch is not None:
        tgt = labels.get(ins.branch)
        succ = [] if tgt is None else [tgt]
        if ins.cond:
            succ.append(j + 1)
        return [s for s in succ if s < len(insts)]
    return [j + 1] if j + 1 < len(insts) else []


def _scan(insts, labels, i, budget, visit):
    """Call visit(j, ws_between) for every instruction j reachable from i
    with fewer than `budget` wait states issued strictly between i and j."""
    seen = {}
    stack = [(s, 0) for s in _successors(insts, labels, i)]
    while stack:
        j, ws = stack.pop()
        if ws >= budget or seen.get(j, budget + 1) <= ws:
            continue
        seen[j] = ws
        if visit(j, ws) is False:
            continue
        nws = ws + insts[j].wait_states
        for s in _successors(insts, labels, j):
            stack.append((s, nws))


def _first_consumers(insts, labels, i, regs, want):
    """(j, wait states) of the first instructions after i that touch `regs`
    (as decided by want(c) -> bool|None: True counts, False stops the path)."""
    found = []

    def visit(j, ws):
        r = want(insts[j])
        if r is True:
            found.append((j, ws))
            return False
        return r is not False
    _scan(insts, labels, i, MAX_WINDOW, visit)
    return found


def calibrate(probe_asm):
    """Bounds observed in the compiler's output for the probe kernels:
    {'raw': {op: n}, 'srcc': {op: n}, 'valu_xdl': n, 'm0_dma': n,
    'valu_sgpr_vmem': n}."""
    funcs, labels = split_functions(probe_asm)
    raw, srcc, valu, m0, sgpr = {}, {}, [], [], []
    for name, insts in funcs.items():
        lab = labels[name]
        for i, p in enumerate(insts):
            if p.is_xdl:
                for j, ws in _first_consumers(
                        insts, lab, i, p.defs,
                        lambda c, p=p: True if _xdl_reads(c, p) else None):
                    d = srcc if _xdl_reads(insts[j], p) == "srcc" else raw
                    d[p.op] = min(d.get(p.op, MAX_WINDOW), ws)
            elif p.is_valu and p.vdefs:
                for j, ws in _first_consumers(
                        insts, lab, i, p.vdefs,
                        lambda c, p=p: True if c.is_xdl and (c.uses & p.vdefs)
                        else (False if c.defs & p.vdefs else None)):
                    valu.append(ws)
            if p.is_valu and p.sdefs:
                for j, ws in _first_consumers(
                        insts, lab, i, p.sdefs,
                        lambda c, p=p: True if c.is_vmem and (c.uses & p.sdefs)
                        else (False if c.is_valu and c.sdefs >= p.sdefs else None)):
                    sgpr.append(ws)
            if p.writes_m0:
                for j, ws in _first_consumers(
                        insts, lab, i, None,
                        lambda c: True if c.reads_m0_dma else (False if c.writes_m0 else None)):
                    m0.append(ws)
    return {"raw": raw, "srcc": srcc, "valu_xdl": min(valu) if valu else None,
            "m0_dma": min(m0) if m0 else None,
            "valu_sgpr_vmem": min(sgpr) if sgpr else None}


def _xdl_reads(c, p):
    """Bound that applies when instruction c follows XDL op p, or None."""
    if c.is_xdl:
        if c.srcab & p.defs:
            return "raw"
        if c.srcc & p.defs:
            return "srcc" if c.srcc == p.defs else "raw"
        return None
    return "raw" if (c.uses | c.defs) & p.defs else None


def check_function(insts, labels, bounds):
    """Violations in one kernel, as human-readable strings."""
    bad = []
    for i, p in enumerate(insts):
        if p.is_xdl:
            if p.op not in bounds["raw"] or p.op not in bounds["srcc"]:
                bad.append(f"[{i}] {p.op}: no bound for this XDL op (extend the probes)")
                continue

            def after_write(j, ws, p=p, i=i):
                c = insts[j]
                kind = _xdl_reads(c, p)
                if kind is not None:
                    n = bounds[kind][p.op]
                    if ws < n:
                        bad.append(f"[{i}] {p.text} -> [{j}] {c.text}: {ws} < {n} wait states")
                    if not c.is_xdl:
                        return False        # a later access re-bases the check
                return True
            _scan(insts, labels, i, max(bounds["raw"][p.op], bounds["srcc"][p.op]), after_write)
        elif p.is_valu and p.vdefs:
            def valu_then_xdl(j, ws, p=p, i=i):
                c = insts[j]
                if c.is_xdl and (c.uses & p.vdefs):
                    bad.append(f"[{i}] {p.text} -> [{j}] {c.text}: {ws} < {bounds['valu_xdl']}")
                return not (c.defs & p.vdefs)
            _scan(insts, labels, i, bounds["valu_xdl"], valu_then_xdl)
        if p.is_valu and p.sdefs:
            def sgpr_then_vmem(j, ws, p=p, i=i):
                c = insts[j]
                if c.is_vmem and (c.uses & p.sdefs):
                    bad.append(f"[{i}] {p.text} -> [{j}] {c.text}: {ws} < "
                               f"{bounds['valu_sgpr_vmem']}")
                return not (c.is_valu and c.sdefs >= p.sdefs)
            _scan(insts, labels, i, bounds["valu_sgpr_vmem"], sgpr_then_vmem)
        if p.writes_m0:
            def m0_then_dma(j, ws, p=p, i=i):
                c = insts[j]
                if c.reads_m0_dma:
                    bad.append(f"[{i}] {p.text} -> [{j}] {c.text}: {ws} < {bounds['m0_dma']}")
                return not c.writes_m0
            _scan(insts, labels, i, bounds["m0_dma"], m0_then_dma)
    return bad


def check_asm(asm_text, bounds, name_filter=None):
    """({kernel symbol: [violations]}, number of XDL ops seen) for the kernels
    whose symbol contains `name_filter` (all kernels if None)."""
    funcs, labels = split_functions(asm_text)
    out, n_xdl = {}, 0
    for name, insts in funcs.items():
        if name_filter and name_filter not in name:
            continue
        n_xdl += sum(1 for x in insts if x.is_xdl)
        out[name] = check_function(insts, labels[name], bounds)
    return out, n_xdl
