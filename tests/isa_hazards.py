"""Static check of gfx950 assembly for loads that are still in flight.

The kernels issue many of their loads from inline asm (LDS reads, buffer loads
into registers) and wait for them with explicit s_waitcnt. The compiler takes
an asm result as available at once, so it may copy it, or reuse its registers
once it considers the value dead, while the hardware is still writing them: the
copy reads stale data, and a late-arriving load can overwrite a register that
meanwhile holds something else (an address, an accumulator). This module finds
such accesses in the compiled code.

Model (per wave, on the control-flow graph of each function, to a fixed point):
  - an outstanding load is (destination registers, counter, age), where age
    counts the younger operations on the same counter;
  - LDS reads return in order, so s_waitcnt lgkmcnt(N) retires every LDS read
    with age >= N; scalar loads return out of order and retire only at
    lgkmcnt(0);
  - vector-memory operations complete in order: s_waitcnt vmcnt(N) retires
    the loads with age >= N;
  - paths join by union, keeping the smaller age.
Any instruction whose operands name a register of an outstanding load is
reported, except a younger load of the same kind into the same registers
(in-order return: it lands last)."""
import re

_REG = re.compile(r"\b([vas])\[(\d+):(\d+)\]|\b([vas])(\d+)\b")
_MAX_AGE = 64


def _regs(text):
    out = set()
    for m in _REG.finditer(text):
        if m.group(1):
            out.update((m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1))
        else:
            out.add((m.group(4), int(m.group(5))))
    return frozenset(out)


def _kind(op, rest):
    """(counter, has a register result, counts as a younger op for its counter's
    in-order returns) of a memory instruction, else None. LDS instructions
    complete in order, and so do vector-memory ones (stores and loads into LDS
    included: on gfx9 vmcnt counts them all)."""
    if op.startswith("ds_"):
        loads = op.startswith(("ds_read", "ds_load")) or op in ("ds_bpermute_b32", "ds_permute_b32", "ds_swizzle_b32")
        return ("lds", loads, True)
    if op.startswith(("s_load", "s_buffer_load")) or op in ("s_memtime", "s_memrealtime"):
        return ("smem", True, False)
    if op.startswith(("buffer_", "global_", "flat_")):
        return ("vmem", "load" in op and " lds" not in rest, True)
    return None


def _functions(asm):
    """{name: [(line number, op, operand text)]} for every function body."""
    funcs, cur = {}, None
    for no, raw in enumerate(asm.split("\n"), 1):
        t = raw.split(";")[0].strip()
        if not t:
            continue
        if t.endswith(":") and not t.startswith("."):
            cur = t[:-1]
            funcs[cur] = []
            continue
        if cur is None:
            continue
        if t.startswith(".Lfunc_end"):
            cur = None
            continue
        if t.endswith(":"):
            funcs[cur].append((no, "label", t[:-1]))
            continue
        if t.startswith("."):
            continue
        op = t.split()[0]
        funcs[cur].append((no, op, t[len(op):]))
    return funcs


def _blocks(body):
    """Basic blocks [(label, [instructions], [successor labels])]."""
    blocks, cur, label = [], [], "<entry>"
    for ins in body:
        no, op, rest = ins
        if op == "label":
            blocks.append([label, cur, None])
            label, cur = rest, []
            continue
        cur.append(ins)
        if op == "s_branch" or op.startswith("s_cbranch") or op == "s_endpgm":
            blocks.append([label, cur, None])
            label, cur = "<after %d>" % no, []
    blocks.append([label, cur, None])
    for i, b in enumerate(blocks):
        succ = []
        last = b[1][-1] if b[1] else None
        nxt = blocks[i + 1][0] if i + 1 < len(blocks) else None
        if last is not None and last[1] == "s_endpgm":
            pass
        elif last is not None and last[1] == "s_branch":
            succ.append(last[2].strip())
        elif last is not None and last[1].startswith("s_cbranch"):
            succ.append(last[2].strip())
            if nxt:
                succ.append(nxt)
        elif nxt:
            succ.append(nxt)
        b[2] = succ
    return blocks


def _transfer(state, ins, report):
    no, op, rest = ins
    if op == "s_waitcnt":
        mv = re.search(r"vmcnt\((\d+)\)", rest)
        ml = re.search(r"lgkmcnt\((\d+)\)", rest)
        out = {}
        for key, (d, ctr, age) in state.items():
            if ctr == "vmem" and mv and age >= int(mv.group(1)):
                continue
            if ctr == "lds" and ml and age >= int(ml.group(1)):
                continue
            if ctr == "smem" and ml and int(ml.group(1)) == 0:
                continue
            out[key] = (d, ctr, age)
        return out
    k = _kind(op, rest)
    ops = rest.split(",")
    dest = _regs(ops[0]) if k and k[1] else frozenset()
    srcs = _regs(",".join(ops[1:])) if k and k[1] else _regs(rest)
    for key, (d, ctr, age) in state.items():
        touched = (srcs & d) or (dest & d and not (k and k[1] and k[0] == ctr and ctr != "smem"))
        if touched and report is not None:
            report.append((no, op + rest, key))
    if not k:
        return state
    out = {}
    for key, (d, ctr, age) in state.items():
        out[key] = (d, ctr, min(age + 1, _MAX_AGE) if ctr == k[0] and k[2] else age)
    if k[1] and dest:
        out[no] = (dest, k[0], 0)
    return out


def _join(a, b):
    out = dict(a)
    for key, v in b.items():
        if key in out:
            out[key] = (v[0], v[1], min(v[2], out[key][2]))
        else:
            out[key] = v
    return out


def hazards(asm):
    """[(function, line, instruction, line of the load)] for the assembly text."""
    found = []
    for name, body in _functions(asm).items():
        blocks = _blocks(body)
        index = {b[0]: i for i, b in enumerate(blocks)}
        entry = [dict() for _ in blocks]
        work = [0]
        seen = set()
        while work:
            i = work.pop()
            st = entry[i]
            for ins in blocks[i][1]:
                st = _transfer(st, ins, None)
            for s in blocks[i][2]:
                j = index.get(s)
                if j is None:
                    continue
                new = _join(entry[j], st)
                if j not in seen or new != entry[j]:
                    seen.add(j)
                    entry[j] = new
                    work.append(j)
        for i, b in enumerate(blocks):
            st, rep = entry[i], []
            for ins in b[1]:
                st = _transfer(st, ins, rep)
            found.extend((name, no, text, load) for no, text, load in rep)
    return found
