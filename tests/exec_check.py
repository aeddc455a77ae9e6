"""Checks, on the gfx950 assembly of this library's own kernels, that every
workgroup barrier runs with the whole wavefront active.

Why: `s_barrier` is a scalar instruction.  A wavefront that reaches it while
some of its lanes are masked off (inside a lane-divergent branch or loop)
arrives for all of its lanes; the masked lanes reach the same barrier again
later, one barrier out of step with every other wavefront, and whatever is
handed through LDS across that barrier is read stale (a ticket loop that did
so copied one chunk forever).  Source rules keep this from happening (loops
around barriers bounded by scalar values, leader work in wave-uniform
branches); this check reads what the compiler made of them.

How: a forward dataflow over each function's control-flow graph.  Lane masks
get symbolic names: "S0" is the EXEC a kernel starts with (every lane), "Z"
the empty mask, and "@L" the EXEC current at line L where an instruction
saves or names it.  The state holds
  ex      the name EXEC equals, or None;
  within  names S with EXEC a subset of S;
  facts   (r, S): EXEC | r == S (a saved mask, an else mask, a loop's
          exited-lanes accumulator);
  vals    (r, S): register pair r holds S;
  subs    (r, S): r is a subset of S (compare results, masks and-ed from
          saved ones);
  symsub  (T, S): mask T is a subset of mask S;
  saved   (S, r, T): while EXEC was S, EXEC | r == T held (restored with S:
          the facts of an enclosing region);
  alias   (@L, S): the mask named @L is S (a mask is always named after the
          line that names it, so that paths reaching the line with different
          names for EXEC agree on it);
  lanes   (sN, slot): sN was last read back from spill slot "vM:L";
  comps   (r, q, S): r | q == S (q and-ed out of a register holding S, r
          the rest by xor: an if's two lane sets saved in two steps).
Scalar registers spilled to VGPR lanes carry their facts through the slot:
half h of pair P written to slot X is the pseudo-register "X#P#h", and a
pair read back from the two slots of one P gets P's facts.

Transfer functions follow the AMDGPU backend's lowering of divergent control
flow: and-saveexec at an if, xor for its else mask, andn2-saveexec at the
else, or at the join, or of a break mask and andn2 at a loop latch, the
same in two steps (mov from EXEC, and, mov to EXEC), and an or-saveexec /
xor pair for an else reached from several places.  What is not followed
drops what was known, and joins intersect, so a barrier reached with
ex != "S0" is reported: the analysis errs towards reporting.
"""

from __future__ import annotations

import re
import subprocess
from dataclasses import dataclass, replace
from functools import lru_cache

S0, Z = "S0", "Z"

_LABEL = re.compile(r"^(\.?[A-Za-z_$][\w.$]*):")
_RANGE = re.compile(r"^s\[(\d+):(\d+)\]$")
_SINGLE = re.compile(r"^s(\d+)$")
_VRANGE = re.compile(r"^v\[(\d+):(\d+)\]$")
_VSINGLE = re.compile(r"^v(\d+)$")

# Scalar instructions whose first operand is read, not written.
_NO_DEST = (
    "s_cmp", "s_bitcmp", "s_cbranch", "s_branch", "s_waitcnt", "s_nop", "s_barrier", "s_setprio",
    "s_sleep", "s_setreg", "s_sendmsg", "s_endpgm", "s_trap", "s_set_gpr_idx", "s_cmpk", "s_dcache",
    "s_icache", "s_ttrace", "s_wait", "s_code_end", "s_denorm", "s_round_mode", "s_sethalt",
    "s_setkill", "s_buffer_atomic", "s_atomic", "s_store", "s_buffer_store",
)


@lru_cache(maxsize=None)
def _sregs(op: str) -> frozenset:
    """Scalar registers an operand names ('s12', 'vcc', 'exec')."""
    op = op.strip()
    if op.startswith("exec"):
        return frozenset({"exec"})
    if op.startswith("vcc"):
        return frozenset({"vcc"})
    m = _RANGE.match(op)
    if m:
        return frozenset(f"s{i}" for i in range(int(m.group(1)), int(m.group(2)) + 1))
    m = _SINGLE.match(op)
    return frozenset({f"s{m.group(1)}"}) if m else frozenset()


def _vregs(op: str) -> list:
    op = op.strip()
    m = _VRANGE.match(op)
    if m:
        return [f"v{i}" for i in range(int(m.group(1)), int(m.group(2)) + 1)]
    return [op] if _VSINGLE.match(op) else []


def _pair(op: str):
    """Canonical name of a 64-bit scalar register operand, or None."""
    op = op.strip()
    if op in ("exec", "vcc"):
        return op
    m = _RANGE.match(op)
    if m and int(m.group(2)) == int(m.group(1)) + 1:
        return op
    return None


@dataclass(frozen=True)
class State:
    ex: object = S0
    within: frozenset = frozenset()
    facts: frozenset = frozenset()
    vals: frozenset = frozenset()
    subs: frozenset = frozenset()
    symsub: frozenset = frozenset()
    saved: frozenset = frozenset()
    alias: frozenset = frozenset()
    lanes: frozenset = frozenset()
    comps: frozenset = frozenset()


@lru_cache(maxsize=1 << 14)
def _amap(alias: frozenset) -> dict:
    return dict(alias)


def _res(st: State, sym):
    return _amap(st.alias).get(sym, sym)


def _sups(st: State, sym):
    """Names known to contain mask `sym` (itself included); None: every name
    (the empty mask)."""
    if sym == Z:
        return None
    return _sups_of(st.symsub, st.alias, sym)


@lru_cache(maxsize=1 << 16)
def _sups_of(symsub: frozenset, alias: frozenset, sym) -> frozenset:
    amap = _amap(alias)
    out = {sym, amap.get(sym, sym), S0}
    grow = True
    while grow:
        grow = False
        for t, s in symsub:
            if (t in out or amap.get(t, t) in out) and s not in out:
                out.add(s)
                grow = True
    out |= {amap.get(s, s) for s in out}
    return frozenset(out)


def _exec_sups(st: State) -> set:
    out = {S0}
    for s in st.within | ({st.ex} if st.ex is not None else set()):
        out |= _sups(st, s) or set()
    return out


def _reg_sups(st: State, r):
    """Names known to contain register pair r (None: every name)."""
    if r is None:
        return {S0}
    if r == "exec":
        return _exec_sups(st)
    out = {S0}
    for p, t in st.vals | st.subs:
        if p == r:
            s = _sups(st, t)
            if s is None:
                return None
            out |= s
    return out


def _cap(a, b):
    if a is None:
        return b
    if b is None:
        return a
    return a & b


def _covers(st: State, r):
    """Name S with EXEC | r == S, or None."""
    if st.ex is not None and _res(st, st.ex) == S0:
        return S0
    for p, s in st.facts:
        if p == r:
            return s
    return None


def _val(st: State, r):
    for p, s in st.vals:
        if p == r:
            return s
    return None


def _meet(xa, xb, ra, rb, syms):
    """Intersection of two sets of tuples whose positions `syms` hold mask
    names: kept where equal as written, else where equal once each side's
    names are resolved (then in resolved form)."""
    if xa == xb:
        return xa
    out = set(xa & xb)

    def res(t, r):
        return tuple(r(v) if k in syms else v for k, v in enumerate(t))

    rb_set = {res(t, rb) for t in xb}
    for t in xa - xb:
        rt = res(t, ra)
        if rt in rb_set:
            out.add(rt)
    return frozenset(out)


def _join(a: State, b: State) -> State:
    ra = lambda v: _res(a, v)
    rb = lambda v: _res(b, v)
    # With EXEC every lane, EXEC | r is every lane for any r.
    fa = a.facts | ({(p, S0) for p, _ in b.facts} if a.ex == S0 else set())
    fb = b.facts | ({(p, S0) for p, _ in a.facts} if b.ex == S0 else set())
    if a.ex == b.ex:
        ex = a.ex
    elif a.ex is not None and b.ex is not None and ra(a.ex) == rb(b.ex):
        ex = ra(a.ex)
    else:
        ex = None
    wa = {(s,) for s in a.within | ({a.ex} if a.ex is not None else set())}
    wb = {(s,) for s in b.within | ({b.ex} if b.ex is not None else set())}
    within = frozenset(t[0] for t in _meet(frozenset(wa), frozenset(wb), ra, rb, (0,)))
    return State(ex, within, _meet(fa, fb, ra, rb, (1,)), _meet(a.vals, b.vals, ra, rb, (1,)),
                 _meet(a.subs, b.subs, ra, rb, (1,)), _meet(a.symsub, b.symsub, ra, rb, (0, 1)),
                 _meet(a.saved, b.saved, ra, rb, (0, 2)), a.alias & b.alias, a.lanes & b.lanes,
                 _meet(a.comps, b.comps, ra, rb, (2,)))


@dataclass
class Insn:
    line: int
    op: str
    args: list


def parse_functions(asm: str):
    """{function symbol: [Insn or local label]} for every function in the file."""
    funcs = {}
    body = None
    code = set(re.findall(r"^\s*\.type\s+([\w.$]+),\s*@function", asm, re.M))
    for i, raw in enumerate(asm.splitlines(), 1):
        line = raw.split(";")[0].rstrip()
        if not line.strip():
            continue
        m = _LABEL.match(line)
        if m:
            name = m.group(1)
            if name.startswith(".Lfunc_end"):
                body = None
            elif not name.startswith("."):
                body = funcs.setdefault(name, []) if name in code else None
            elif body is not None:
                body.append(name)
            continue
        if body is None:
            continue
        parts = line.strip().split(None, 1)
        if parts[0].startswith("."):
            continue
        args = [x.strip() for x in parts[1].split(",")] if len(parts) > 1 else []
        body.append(Insn(i, parts[0], args))
    return {k: v for k, v in funcs.items() if any(isinstance(x, Insn) for x in v)}


def _drop(st: State, regs) -> State:
    """Forget everything about register pairs that overlap `regs`."""
    def hit(p):
        return not _sregs(p).isdisjoint(regs)

    return replace(st, facts=frozenset(f for f in st.facts if not hit(f[0])),
                   vals=frozenset(v for v in st.vals if not hit(v[0])),
                   subs=frozenset(v for v in st.subs if not hit(v[0])),
                   saved=frozenset(s for s in st.saved if not hit(s[1])),
                   lanes=frozenset(x for x in st.lanes if x[0] not in regs),
                   comps=frozenset(c for c in st.comps if not hit(c[0]) and not hit(c[1])))


def _name_exec(st: State, line: int):
    """The current EXEC named after this line, with what is known of it kept
    for when it is restored: (state, name)."""
    sym = f"@{line}"
    # A new instance of this line's mask: forget the previous one's.
    st = replace(st, within=frozenset(s for s in st.within if s != sym),
                 facts=frozenset(f for f in st.facts if f[1] != sym),
                 vals=frozenset(v for v in st.vals if v[1] != sym),
                 subs=frozenset(v for v in st.subs if v[1] != sym),
                 symsub=frozenset(x for x in st.symsub if sym not in x),
                 saved=frozenset(s for s in st.saved if s[0] != sym and s[2] != sym),
                 alias=frozenset(x for x in st.alias if sym not in x),
                 comps=frozenset(c for c in st.comps if c[2] != sym))
    bounds = _exec_sups(st)
    stash = {(sym, p, t) for p, t in st.facts}
    alias = set(st.alias)
    if st.ex is not None:
        stash |= {(sym, p, t) for s, p, t in st.saved if s == st.ex}
        alias.add((sym, _res(st, st.ex)))
    return replace(st, ex=st.ex if st.ex is not None else sym, within=st.within | {sym},
                   symsub=st.symsub | {(sym, b) for b in bounds if b != sym},
                   saved=st.saved | stash, alias=frozenset(alias)), sym


def _restore(st: State, sym) -> State:
    """EXEC is again the mask named `sym`: reinstate what was known then."""
    target = _res(st, sym)
    facts = frozenset((p, t) for s, p, t in st.saved if s in (sym, target))
    st = replace(st, ex=target, facts=facts)
    return replace(st, within=frozenset(_sups(st, target) or ()))


def _kept_on_shrink(st: State, bound):
    """Facts EXEC | r == S that survive EXEC becoming a subset of names
    `bound`: those with r == S and EXEC inside S."""
    out = set()
    for p, t in st.facts:
        v = _val(st, p)
        if v is not None and _res(st, v) == _res(st, t) and _res(st, t) in bound:
            out.add((p, t))
    return frozenset(out)


def _grow_exec(st: State, src) -> State:
    """EXEC := EXEC | src."""
    if src == "-1":
        return _restore(st, S0)
    sp = _pair(src)
    cov = _covers(st, sp)
    if cov is not None:
        return _restore(st, cov)
    v = _val(st, sp)
    if v is not None and v != Z and _res(st, v) in _exec_sups(st):
        return _restore(st, v)  # EXEC inside v, and v added: EXEC == v
    src_sups = _reg_sups(st, sp)
    within = _cap(_exec_sups(st), src_sups)
    facts = frozenset((p, t) for p, t in st.facts if src_sups is None or _res(st, t) in src_sups)
    return replace(st, ex=None, within=frozenset(within), facts=facts)


def _shrink(st: State, extra=(), bound=None) -> State:
    """EXEC became a subset of the names `bound` (of the old EXEC if None)."""
    within = _exec_sups(st) if bound is None else set(bound)
    return replace(st, ex=None, within=frozenset(within), facts=_kept_on_shrink(st, within) | frozenset(extra))


def _transfer(st: State, ins: Insn) -> State:
    op, a = ins.op, ins.args
    dst = a[0] if a else ""
    d = _pair(dst)

    # ---- writes to EXEC
    if op == "s_and_saveexec_b64":
        st, sym = _name_exec(st, ins.line)
        st = _drop(st, _sregs(dst))
        st = replace(st, vals=st.vals | {(d, sym)})
        return _shrink(st, {(d, sym)})
    if op in ("s_andn2_saveexec_b64", "s_andn1_saveexec_b64"):
        src = _pair(a[1])
        cov, src_sups = _covers(st, src), _reg_sups(st, src)
        st, sym = _name_exec(st, ins.line)
        st = _drop(st, _sregs(dst))
        st = replace(st, vals=st.vals | {(d, sym)})
        # new EXEC == src & ~old, d == old: EXEC | d == src | old.
        return _shrink(st, {(d, cov)} if cov is not None else (), bound=src_sups or {S0})
    if op == "s_or_saveexec_b64":
        st, sym = _name_exec(st, ins.line)
        src = a[1].strip()
        st = _drop(st, _sregs(dst) - _sregs(src))
        st = replace(st, vals=st.vals | {(d, sym)})
        return _grow_exec(st, src)
    if dst == "exec" and op == "s_or_b64" and len(a) == 3 and "exec" in (a[1], a[2]):
        return _grow_exec(st, a[2] if a[1] == "exec" else a[1])
    if dst == "exec" and op == "s_andn2_b64" and len(a) == 3 and a[1] == "exec":
        other = _pair(a[2])
        cov = _covers(st, other)
        # (EXEC & ~r) | r == EXEC | r.
        return _shrink(st, {(other, cov)} if cov is not None else ())
    if dst == "exec" and op == "s_and_b64" and "exec" in a[1:3]:
        return _shrink(st)
    if op.startswith("v_cmpx"):
        return _shrink(st)
    if dst == "exec" and op == "s_xor_b64" and len(a) == 3 and "exec" in a[1:3]:
        # EXEC ^ r lies inside EXEC | r, and (EXEC ^ r) | r == EXEC | r.
        r = _pair(a[2] if a[1] == "exec" else a[1])
        cov = _covers(st, r)
        return _shrink(st, {(r, cov)} if cov is not None else (),
                       bound=_cap(_exec_sups(st), _reg_sups(st, r)) or {S0})
    if dst == "exec" and op == "s_mov_b64":
        src = a[1].strip()
        if src == "-1":
            return _restore(st, S0)
        sp = _pair(src)
        v = _val(st, sp)
        if v is not None and v != Z:
            return _restore(st, v)
        # EXEC := q, one of two lane sets r | q == S: EXEC | r == S.
        extra = {(r, t) for r, q, t in st.comps if q == sp}
        return _shrink(st, extra, bound=_reg_sups(st, sp) or {S0})
    if "exec" in _sregs(dst) and not op.startswith(_NO_DEST):
        return replace(st, ex=None, within=frozenset(), facts=frozenset())

    # ---- scalar registers spilled to VGPR lanes
    if op == "v_writelane_b32" and len(a) == 3:
        slot = f"{a[0]}:{a[2]}"
        st = _forget_slot(st, slot)
        k = _sregs(a[1])
        if len(k) == 1 and next(iter(k)) not in ("exec", "vcc"):
            n = int(next(iter(k))[1:])
            pair, h = f"s[{n & ~1}:{(n & ~1) + 1}]", n & 1
            tag = f"{slot}#{pair}#{h}"
            st = replace(st, facts=st.facts | {(tag, t) for p, t in st.facts if p == pair},
                         vals=st.vals | {(tag, t) for p, t in st.vals if p == pair},
                         subs=st.subs | {(tag, t) for p, t in st.subs if p == pair})
        return st
    if op == "v_readlane_b32" and len(a) == 3:
        k = _sregs(a[0])
        st = _drop(st, k)
        if len(k) != 1 or next(iter(k)) in ("exec", "vcc"):
            return st
        reg = next(iter(k))
        st = replace(st, lanes=st.lanes | {(reg, f"{a[1]}:{a[2]}")})
        n = int(reg[1:])
        lo, hi = f"s{n & ~1}", f"s{(n & ~1) + 1}"
        src = dict(st.lanes)
        if lo in src and hi in src:
            q = f"s[{n & ~1}:{(n & ~1) + 1}]"
            sl, sh = src[lo], src[hi]

            def back(xs):
                out = set()
                for name, t in xs:
                    if name.startswith(sl + "#") and name.endswith("#0"):
                        pair = name[len(sl) + 1:-2]
                        if (f"{sh}#{pair}#1", t) in xs:
                            out.add((q, t))
                return out

            st = replace(st, facts=st.facts | back(st.facts), vals=st.vals | back(st.vals),
                         subs=st.subs | back(st.subs))
        return st
    if op.startswith("v_") and a:
        for v in _vregs(a[0]):
            st = _forget_slot(st, f"{v}:", prefix=True)

    # ---- other writes to scalar registers
    written = set()
    if op.startswith("s_") and not op.startswith(_NO_DEST):
        written = _sregs(dst)
    elif op.startswith("v_cmp"):
        written = _sregs(dst)
    elif op.startswith("v_"):
        # VOP3 carry-outs and the like: any scalar register among the first
        # two operands is taken as written.
        for x in a[:2]:
            written |= _sregs(x)
    if not written:
        return st
    if op.startswith("v_cmp") and d:
        # Compare results are zero in inactive lanes: inside EXEC.
        bounds = _exec_sups(st)
        st = _drop(st, written)
        return replace(st, subs=st.subs | {(d, b) for b in bounds if b != S0})
    if not d or op.startswith("v_"):
        return _drop(st, written)
    srcs = [x.strip() for x in a[1:]]
    sp = [_pair(x) for x in srcs]
    if op == "s_or_b64" and len(a) == 3 and d in sp:
        # d |= x (a break mask gathering lanes of EXEC): EXEC | d == S still
        # holds where x lies inside S.
        x = sp[1] if sp[0] == d else sp[0]
        xs = _reg_sups(st, x)
        facts = frozenset((p, t) for p, t in st.facts if p != d or xs is None or _res(st, t) in xs)
        subs_d = _cap(_reg_sups(st, d), xs) or set()
        st = replace(st, facts=facts, vals=frozenset(v for v in st.vals if v[0] != d),
                     subs=frozenset(v for v in st.subs if v[0] != d),
                     lanes=frozenset(v for v in st.lanes if v[0] not in written))
        return replace(st, subs=st.subs | {(d, b) for b in subs_d if b != S0})
    if op == "s_xor_b64" and len(a) == 3 and "exec" not in srcs and sp[0] and sp[1]:
        # d = x ^ q with x holding S and q inside S: d | q == S.
        comps = set()
        for x, q in ((sp[0], sp[1]), (sp[1], sp[0])):
            v = _val(st, x)
            if v is not None and v != Z and _res(st, v) in (_reg_sups(st, q) or {_res(st, v)}):
                comps.add((d, q, v))
        st = _drop(st, written)
        return replace(st, comps=st.comps | frozenset(c for c in comps if c[1] != d))
    if op == "s_xor_b64" and len(a) == 3 and "exec" in srcs:
        # The else mask of an if/else: EXEC | (r ^ EXEC) == EXEC | r.
        r = sp[1] if srcs[0] == "exec" else sp[0]
        cov = _covers(st, r)
        bound = _cap(_exec_sups(st), _reg_sups(st, r)) or set()
        st = _drop(st, written)
        return replace(st, facts=st.facts | ({(d, cov)} if cov is not None else set()),
                       subs=st.subs | {(d, b) for b in bound if b != S0})
    if op == "s_mov_b64" and srcs[0] == "exec":
        st = _drop(st, written)
        st, sym = _name_exec(st, ins.line)
        return replace(st, facts=st.facts | {(d, sym)}, vals=st.vals | {(d, sym)})
    if op == "s_mov_b64" and srcs[0] == "0":
        # EXEC | 0 == EXEC: a break-mask accumulator may start here.
        st = _drop(st, written)
        st, sym = _name_exec(st, ins.line)
        return replace(st, facts=st.facts | {(d, sym)}, vals=st.vals | {(d, Z)})
    if op == "s_mov_b64" and srcs[0] == "-1":
        st = _drop(st, written)
        return replace(st, facts=st.facts | {(d, S0)}, vals=st.vals | {(d, S0)})
    if op == "s_mov_b64" and sp[0]:
        cov, val, rs = _covers(st, sp[0]), _val(st, sp[0]), _reg_sups(st, sp[0])
        st = _drop(st, written)
        return replace(st, facts=st.facts | ({(d, cov)} if cov is not None else set()),
                       vals=st.vals | ({(d, val)} if val is not None else set()),
                       subs=st.subs | {(d, b) for b in (rs or ()) if b != S0})
    if op in ("s_and_b64", "s_andn2_b64") and len(a) == 3:
        # d lies inside whatever x (or, for and, y) lies inside.
        bound = set(_reg_sups(st, sp[0]) or ())
        if op == "s_and_b64":
            bound |= _reg_sups(st, sp[1]) or set()
        st = _drop(st, written)
        return replace(st, subs=st.subs | {(d, b) for b in bound if b != S0})
    if op == "s_or_b64" and len(a) == 3:
        bound = _cap(_reg_sups(st, sp[0]), _reg_sups(st, sp[1])) or set()
        st = _drop(st, written)
        return replace(st, subs=st.subs | {(d, b) for b in bound if b != S0})
    return _drop(st, written)


def _forget_slot(st: State, slot: str, prefix=False) -> State:
    """Forget the pseudo-registers of a spill slot (or of every slot of a VGPR)."""
    key = slot if prefix else slot + "#"

    def hit_lane(s):
        return s.startswith(slot) if prefix else s == slot

    if not any(n.startswith(key) for n, _ in st.facts | st.vals | st.subs) and \
            not any(hit_lane(x[1]) for x in st.lanes):
        return st
    return replace(st, facts=frozenset(f for f in st.facts if not f[0].startswith(key)),
                   vals=frozenset(v for v in st.vals if not v[0].startswith(key)),
                   subs=frozenset(v for v in st.subs if not v[0].startswith(key)),
                   lanes=frozenset(x for x in st.lanes if not hit_lane(x[1])))


def _empty(st: State) -> State:
    """EXEC == 0 (an exec-zero branch taken, or an exec-nonzero one not):
    EXEC | r == r, and EXEC lies inside every mask."""
    names = {t for _, t in st.facts | st.vals | st.subs} - {Z}
    facts = st.facts | frozenset((p, t) for p, t in st.vals if t != Z)
    vals = st.vals | st.facts
    return replace(st, ex=None, within=st.within | frozenset(names), facts=facts, vals=vals)


def _blocks(body):
    blocks = []
    cur = [None, []]
    for item in body:
        if isinstance(item, str):
            blocks.append(cur)
            cur = [item, []]
            continue
        cur[1].append(item)
        if item.op.startswith(("s_branch", "s_cbranch", "s_endpgm", "s_setpc")):
            blocks.append(cur)
            cur = [None, []]
    blocks.append(cur)
    return [b for b in blocks if b[0] is not None or b[1]]


def solve(body, max_iter=200000):
    """Basic blocks of a function and the dataflow state at entry to each."""
    blocks = _blocks(body)
    index = {b[0]: i for i, b in enumerate(blocks) if b[0] is not None}

    def succs(i, out):
        insns = blocks[i][1]
        last = insns[-1] if insns else None
        if last is not None and last.op.startswith(("s_endpgm", "s_setpc")):
            return []
        if last is not None and last.op.startswith(("s_branch", "s_cbranch")):
            res = []
            tgt = index.get(last.args[0]) if last.args else None
            if tgt is None:
                raise ValueError(f"branch target not found on line {last.line}: {last.args}")
            # With every lane active EXEC is not zero: an exec-zero branch is
            # not taken, an exec-nonzero one always is.
            full = out.ex is not None and _res(out, out.ex) == S0
            if not (full and last.op == "s_cbranch_execz"):
                res.append((tgt, _empty(out) if last.op == "s_cbranch_execz" else out))
            if last.op != "s_branch" and i + 1 < len(blocks) and not (full and last.op == "s_cbranch_execnz"):
                res.append((i + 1, _empty(out) if last.op == "s_cbranch_execnz" else out))
            return res
        return [(i + 1, out)] if i + 1 < len(blocks) else []

    inn = {0: State()}
    work = [0]
    n = 0
    while work:
        n += 1
        if n > max_iter:
            raise RuntimeError("exec-mask dataflow did not converge")
        i = work.pop()
        st = inn[i]
        for ins in blocks[i][1]:
            st = _transfer(st, ins)
        for j, s in succs(i, st):
            old = inn.get(j)
            new = s if old is None else _join(old, s)
            if old is None or new != old:
                inn[j] = new
                work.append(j)
    return blocks, inn


def check_function(body):
    """Barriers reached with EXEC not known to be every lane: [(asm line, ex)]."""
    blocks, inn = solve(body)
    bad = []
    for i, (_, insns) in enumerate(blocks):
        if i not in inn:
            continue
        st = inn[i]
        for ins in insns:
            if ins.op == "s_barrier" and (st.ex is None or _res(st, st.ex) != S0):
                bad.append((ins.line, st.ex))
            st = _transfer(st, ins)
    return bad


def check_asm(asm: str):
    """({function: [(line, ex)]} for functions with a barrier under a partial
    EXEC, barriers checked, functions checked)."""
    funcs = parse_functions(asm)
    out = {}
    n = 0
    for name, body in funcs.items():
        n += sum(1 for x in body if isinstance(x, Insn) and x.op == "s_barrier")
        bad = check_function(body)
        if bad:
            out[name] = bad
    return out, n, len(funcs)


def device_asm(hipcc: str, src: str, flags) -> str:
    """gfx950 assembly of one source file (device code only)."""
    r = subprocess.run([hipcc, *flags, "--cuda-device-only", "-S", src, "-o", "-"], capture_output=True,
                       text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed for {src}:\n{r.stderr[-4000:]}")
    return r.stdout
