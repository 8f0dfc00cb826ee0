"""A check of the generated gfx950 assembly, run by the build.

The compiler lowers a divergent `if` to: save the execution mask, narrow it
to the lanes that take the branch, `s_cbranch_execz` over the body when no
lane does, and at the join point `s_or_b64 exec, exec, <saved>` to restore
every lane.  A vector instruction placed between the join label and that
restore runs only on the lanes that took the branch.  Code of the body may
legitimately sit there, but a register copy that the register allocator
placed there for a value every lane needs (seen in one build of the
key-major kernel: four `v_accvgpr_write` copies of live accumulator values,
so lanes whose column was past head_dim kept a stale accumulator) silently
corrupts results.  The check lists every such instruction in a join block
that is the target of an `s_cbranch_execz` which narrowed the mask on its way
there; the build refuses a library with any, so that a miscompile of this
kind is caught before it runs.

An `s_cbranch_execz` can also be a plain guard that skips a block when no
lane is active, with the mask left as it was (the compiler emits one before
the zero-fill of a loop's results when the loop ran no trip): its target is
not a join of a divergent `if` and needs no restore, so a branch whose
straight run of code (back to the previous label or unconditional branch)
writes no execution mask marks no join."""
from __future__ import annotations

import re

_FUNC = re.compile(r"^(_Z\S+):")
_LABEL = re.compile(r"^(\.LBB\d+_\d+):")
_EXECZ = re.compile(r"s_cbranch_execz (\.LBB\d+_\d+)")
_RESTORE = re.compile(r"^s_or_b64 exec, exec,")
# an instruction that writes the execution mask
_EXEC_WRITE = re.compile(r"^s_\w*saveexec\w*\s|^s_\w+ exec,")


def _narrows(body, k):
    """Whether the straight run of code that ends in the branch at body[k]
    writes the execution mask."""
    for t in reversed(body[:k]):
        t = t.strip()
        if _EXEC_WRITE.match(t):
            return True
        if _LABEL.match(t) or t.startswith(("s_branch", "s_endpgm", "s_setpc")):
            return False
    return False
# vector instructions that do not depend on the execution mask
_MASK_FREE = re.compile(r"^v_(readlane|writelane|readfirstlane)")


def scan(asm_text: str):
    """[(function, line number, [instructions])] of vector instructions found
    between a join label and the restore of the execution mask."""
    lines = asm_text.split("\n")
    starts = [(i, m.group(1)) for i, l in enumerate(lines) for m in [_FUNC.match(l)] if m]
    starts.append((len(lines), None))
    found = []
    for (a, name), (b, _) in zip(starts, starts[1:]):
        body = lines[a:b]
        joins = {m.group(1) for k, l in enumerate(body) for m in [_EXECZ.search(l)]
                 if m and _narrows(body, k)}
        for k, line in enumerate(body):
            m = _LABEL.match(line)
            if not m or m.group(1) not in joins:
                continue
            prefix = []
            for t in body[k + 1:]:
                t = t.strip()
                if not t or t.startswith(";"):
                    continue
                if _RESTORE.match(t):
                    break
                if _LABEL.match(t) or t.startswith(("s_cbranch", "s_branch", "s_endpgm")):
                    prefix = []
                    break
                prefix.append(t)
            bad = [t for t in prefix if t.startswith("v_") and not _MASK_FREE.match(t)]
            if bad:
                found.append((name, a + k + 1, bad))
    return found
