"""Checks the K-loops of compiled GEMM kernels for waits on the vector-memory
counter that the compiler inserts before a step's first matrix instruction.

The tile loops stage their operands with global-to-LDS loads written as
inline asm and count them themselves (an explicit wait at the end of each
step); the compiler's own wait insertion does not see those loads.  It adds a
wait of its own when it believes that a load of its own, with a register
result, may still be in flight when the loop reuses that register: a copy
whose software pipeline ends with a prefetch on some path, a poll or an
atomic whose result stays pending.  Such a wait sits at the top of every
step, counts only the loads the compiler knows of, and so also waits for the
stage loads that should stay in flight: the prefetch is lost without any
change in results (a dispatch GEMM loop carried five of them, an AG-GEMM
loop one).

`kloop_waits(asm)` returns, per function, the waits found before the first
MFMA of each innermost loop that contains MFMAs.
"""

import re

from tests.exec_check import Insn, parse_functions

_BRANCH = re.compile(r"s_(cbranch_\w+|branch)$")


def _loops(body):
    """(start, end) index pairs of the backward branches' loops of a body."""
    labels = {x: i for i, x in enumerate(body) if isinstance(x, str)}
    out = []
    for i, x in enumerate(body):
        if isinstance(x, Insn) and _BRANCH.match(x.op) and x.args and x.args[0] in labels:
            j = labels[x.args[0]]
            if j < i:
                out.append((j, i))
    return out


def _has_mfma(body, a, b):
    return any(isinstance(x, Insn) and x.op.startswith("v_mfma") for x in body[a:b + 1])


def kloop_waits(asm: str):
    """{function: [(first line of the loop, [wait operands])]} for innermost
    MFMA loops with a vmcnt wait ahead of their first MFMA, and the number of
    such loops checked."""
    bad = {}
    checked = 0
    for name, body in parse_functions(asm).items():
        loops = [(a, b) for a, b in _loops(body) if _has_mfma(body, a, b)]
        inner = [(a, b) for a, b in loops
                 if not any((c, d) != (a, b) and a <= c and d <= b for c, d in loops)]
        for a, b in inner:
            checked += 1
            waits = []
            for x in body[a:b + 1]:
                if not isinstance(x, Insn):
                    continue
                if x.op.startswith("v_mfma"):
                    break
                if x.op == "s_waitcnt" and any(arg.startswith("vmcnt") for arg in x.args[0].split()):
                    waits.append(x.args[0])
            if waits:
                first = next(x.line for x in body[a:b + 1] if isinstance(x, Insn))
                bad.setdefault(name, []).append((first, waits))
    return bad, checked
