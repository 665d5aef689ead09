"""Check the hand-placed waits of the streaming tile loads in generated code.

The decode kernel issues its K/V tile loads from inline assembly (marked
``; tile load``) and waits for them with hand-written ``s_waitcnt vmcnt(N)``
(marked ``; tile wait <registers>``).  The compiler does not know these
registers are pending, so this scan of the device assembly proves, for every
kernel, that between a tile load and the wait that retires it:

* no other instruction reads or writes the load's destination registers;
* no compiler-issued vector memory instruction (a load, a store, a register
  spill) is issued: vmcnt would count it and weaken the hand-placed counts;
* each wait's count retires the registers the wait names (loads complete in
  issue order, so vmcnt(N) retires all but the newest N);
* where control-flow paths meet (a loop head, the join after a branch), the
  loads in flight agree, or else only a vmcnt(0) wait follows.

The function is split into basic blocks and the loads in flight at each
block's entry are found by iterating to a fixed point over the control-flow
graph; the checks then run over every block from its entry state.
"""

import re
import sys

_VREG = re.compile(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b")
_VMEM = re.compile(r"^(buffer_|global_|flat_|scratch_)")
_BRANCH = re.compile(r"^s_(cbranch_\w+|branch)\s+(\.LBB\w+)")
_LABEL = re.compile(r"^(\.LBB\w+):")


def _regs(text):
    out = set()
    for a, b, c in _VREG.findall(text):
        if c:
            out.add(int(c))
        else:
            out.update(range(int(a), int(b) + 1))
    return out


class _State:
    """Tile loads in flight: a list of register sets, oldest first; ``ordered``
    is False after paths with different in-flight loads merged."""

    def __init__(self, loads=(), ordered=True):
        self.loads = [frozenset(x) for x in loads]
        self.ordered = ordered

    def copy(self):
        return _State(self.loads, self.ordered)

    def key(self):
        return (tuple(self.loads), self.ordered)

    def pending(self):
        return set().union(*self.loads) if self.loads else set()

    @staticmethod
    def merge(states):
        states = [s for s in states if s is not None]
        if not states:
            return None
        first = states[0]
        if all(s.key() == first.key() for s in states):
            return first.copy()
        regs = frozenset().union(*(s.pending() for s in states))
        n = max(len(s.loads) for s in states)
        # unordered: keep the largest count, every register counts as pending
        return _State([regs] + [frozenset()] * (n - 1), ordered=False)


def _blocks(lines):
    """Split a function into basic blocks: (label, [(line_no, text, in_asm)],
    successor labels, falls_through)."""
    blocks = []
    cur = {"label": None, "ins": [], "succ": [], "falls": True}
    in_asm = False

    def close(nxt_label):
        nonlocal cur
        blocks.append(cur)
        cur = {"label": nxt_label, "ins": [], "succ": [], "falls": True}

    for ln, raw in enumerate(lines):
        t = raw.strip()
        if t.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if t.startswith(";;#ASMEND"):
            in_asm = False
            continue
        m = _LABEL.match(t)
        if m:
            close(m.group(1))
            continue
        if not t or t.startswith(";") or t.startswith("."):
            continue
        cur["ins"].append((ln, t, in_asm))
        if in_asm:
            continue
        body = t.split(";", 1)[0].strip()
        b = _BRANCH.match(body)
        if b:
            cur["succ"].append(b.group(2))
            if b.group(1) == "branch":
                cur["falls"] = False
            close(None)
        elif body.split() and body.split()[0] in ("s_endpgm", "s_setpc_b64", "s_trap"):
            cur["falls"] = False
            close(None)
    blocks.append(cur)
    return blocks


def _run_block(name, block, state, problems):
    """Simulate one block from its entry state; append problems if given."""
    state = state.copy()
    for ln, t, in_asm in block["ins"]:
        if in_asm and "; tile load" in t:
            dest = _regs(t.split(",")[0])
            if problems is not None and dest & state.pending():
                problems.append(f"{name}:{ln}: tile load into a register still in flight: {t}")
            state.loads.append(frozenset(dest))
            continue
        if in_asm and "; tile wait" in t:
            n = int(re.search(r"vmcnt\((\d+)\)", t).group(1))
            if n == 0:
                state = _State()
                continue
            if not state.ordered:
                if problems is not None:
                    problems.append(f"{name}:{ln}: vmcnt({n}) where paths with different loads "
                                    f"in flight meet: {t}")
                # at most n loads remain, but any register may be among them
                if len(state.loads) > n:
                    state = _State([state.pending()] + [frozenset()] * (n - 1), ordered=False)
                continue
            state.loads = state.loads[-n:]
            named = _regs(t.split("; tile wait", 1)[1])
            if problems is not None and named & state.pending():
                problems.append(f"{name}:{ln}: wait does not retire the registers it names: {t}")
            continue
        if in_asm or problems is None or not state.loads:
            continue
        body = t.split(";", 1)[0].strip()
        if not body:
            continue
        if _VMEM.match(body.split()[0]):
            problems.append(f"{name}:{ln}: vector memory instruction while tile loads are "
                            f"in flight: {t}")
        hit = _regs(body) & state.pending()
        if hit:
            problems.append(f"{name}:{ln}: touches in-flight tile registers {sorted(hit)}: {t}")
    return state


def check_function(name, lines, max_rounds=50):
    """Return a list of problems found in one function's assembly lines."""
    blocks = _blocks(lines)
    index = {b["label"]: i for i, b in enumerate(blocks) if b["label"]}
    preds = [[] for _ in blocks]
    for i, b in enumerate(blocks):
        for tgt in b["succ"]:
            if tgt not in index:
                return [f"{name}: branch to unknown label {tgt}"]
            preds[index[tgt]].append(i)
        if b["falls"] and i + 1 < len(blocks):
            preds[i + 1].append(i)
    entry = [None] * len(blocks)
    exit_ = [None] * len(blocks)
    entry[0] = _State()
    for _ in range(max_rounds):
        changed = False
        for i, b in enumerate(blocks):
            st = entry[0] if i == 0 else _State.merge([exit_[p] for p in preds[i]])
            if st is None:
                continue
            if entry[i] is None or st.key() != entry[i].key():
                entry[i] = st
                changed = True
            out = _run_block(name, b, st, None)
            if exit_[i] is None or out.key() != exit_[i].key():
                exit_[i] = out
                changed = True
        if not changed:
            break
    else:
        return [f"{name}: in-flight loads do not settle (a loop that keeps loading?)"]
    problems = []
    for i, b in enumerate(blocks):
        if entry[i] is not None:
            _run_block(name, b, entry[i], problems)
    return problems


def check_assembly(text):
    """Check every function in a device assembly file; return (n_checked, problems)."""
    problems = []
    n = 0
    for m in re.finditer(r"^(_Z\w+):", text, re.M):
        name = m.group(1)
        end = text.find(".Lfunc_end", m.end())
        body = text[m.end():end].splitlines()
        if not any("; tile load" in l for l in body):
            continue
        n += 1
        problems += check_function(name, body)
    return n, problems


if __name__ == "__main__":
    n, probs = check_assembly(open(sys.argv[1]).read())
    print(f"{n} functions with tile loads checked")
    for p in probs:
        print(p)
    sys.exit(1 if probs else 0)
