"""What the library's executor can run as one launch: a model of its
capacity, kept on the test side.

The oracle (oracle/partition.py, oracle/search.py) holds only the rules of
the pages: TVM's three fusion phases with the sink-only reduction, the
opaque barrier and the op and argument limits; DisCo's validity of a plan
(acyclic, no fused opaque op); and the row-resident extension's merge of a
reduction with its readers (convex, within the limits).  Which of those
groupings one kernel launch can actually hold is a property of the
executor, not of the pages.  The tests compose the two: every merge and
every grouping the oracle makes must also pass `group_ok` below, the way
every merge the library makes must compile.

`group_ok` is pinned against the library's own account of each group it
runs (tests/test_capacity.py): the stage count and the LDS bytes that
fuse_plan_group_geometry reports for random valid groupings equal what
`layout` predicts from the shapes and the dataflow alone.

The executor (kernels.hip, isa.h) runs a group on one [R,C] domain:
  * every tensor it touches broadcasts to [R,C]; its reductions read
    [R,C] values and make per-row [R,1] results;
  * element stages: an op runs in the stage of its latest input, a
    reduction's result is readable one stage later; at most MAX_STAGES
    stages and at most one reduction ending each;
  * column ops ([1,C] results) run before any reduction, in stage 0; row
    ops ([R,1] results) and column ops read only their own kind (a column
    op may also read a [1,1] input); a reduction's result read inside the
    group is a per-row value;
  * paired reductions share a stage: a row mean followed by the row mean
    of the squared deviations from it, or a row max followed by the row sum
    of exp(x - max), over one input whose deviations and squares (or
    exponentials) nothing else reads, run as one pass; the two element ops
    between them are not run;
  * at most MAX_SLOTS tensors in memory, MAX_LDS_ROW per-row and
    MAX_LDS_COL per-column operands held in LDS;
  * a transpose, reshape, tuple or concat of two tensors is an addressed
    load of tensors in memory: its inputs are not made in the group and no
    other op of the group reads them (nor their sources, below), a join (a
    tuple or a concat of two) of column values is not run, and no move
    reads a u8 tensor except a reshape;
  * a transpose or reshape whose value only a join of the group reads,
    that is no graph output and keeps its source's dtype, is folded into
    that join: the join reads the move's source at the move's addressing
    (one source at two addressings is not run), and the move is not run;
  * a concat of one tuple is a copy of the tuple's value.
"""
from __future__ import annotations

from typing import Dict, Set

from oracle import partition as pt
from oracle.evaluate import norm_shape

MAX_STAGES = 4
MAX_SLOTS = 16
MAX_LDS_ROW = 8
MAX_LDS_COL = 4
REDUCES = ("row_sum", "row_mean", "row_max")


def is_join(o) -> bool:
    return o.op == "tuple" or (o.op == "concat" and len(o.inputs) == 2)


def is_gather(o) -> bool:
    return o.op in ("transpose", "reshape") or is_join(o)


def folded(graph, members: Set[int]):
    """The moves folded into a join of the group: ({moved value: (source,
    (row stride, column stride))}, the members left to run)."""
    made = {graph.ops[i].output for i in members}
    fold, kept = {}, set()
    for i in sorted(members):
        o = graph.ops[i]
        if (o.op in ("transpose", "reshape") and o.inputs[0] not in made
                and graph.tensors[o.output].role != "out"
                and graph.tensors[o.inputs[0]].dtype == graph.tensors[o.output].dtype):
            readers = [j for j, q in enumerate(graph.ops) for t in q.inputs if t == o.output]
            if len(readers) == 1 and readers[0] in members and is_join(graph.ops[readers[0]]):
                x = o.inputs[0]
                if o.op == "transpose":
                    st = (1, norm_shape(graph.tensors[x].shape)[1])
                else:
                    r, c = norm_shape(graph.tensors[o.output].shape)
                    st = (0 if r == 1 else c, 1)
                fold[o.output] = (x, st)
                continue
        kept.add(i)
    return fold, kept


def gathers_ok(graph, members: Set[int], fold) -> bool:
    """A move or a join runs inside a group only as a load: its inputs come
    from memory and no other op of the group reads them or their sources;
    a join reads each source at one addressing."""
    produced = {graph.ops[i].output for i in members}

    def src(t):
        return fold[t][0] if t in fold else t

    def side(t):
        if t in fold:
            return fold[t]
        r, c = norm_shape(graph.tensors[t].shape)
        return (t, (0 if r == 1 else c, 1))
    for i in members:
        o = graph.ops[i]
        if not is_gather(o):
            continue
        for t in o.inputs:
            if t in produced:
                return False
            if any(u == t or src(u) == src(t) for j in members if j != i for u in graph.ops[j].inputs):
                return False
        if o.op != "reshape" and graph.tensors[o.inputs[0]].dtype == "u8":
            return False
        if is_join(o):
            (sa, la), (sb, lb) = side(o.inputs[0]), side(o.inputs[1])
            if sa == sb and la != lb:
                return False
    return True


def pairs(graph, members: Set[int]):
    """Paired reductions of a group: ({second: first}, the element ops the
    paired pass absorbs)."""
    made = {graph.ops[i].output: i for i in members}
    readers: Dict[int, int] = {}
    for o in graph.ops:
        for t in o.inputs:
            readers[t] = readers.get(t, 0) + 1
    first_of: Dict[int, int] = {}
    taken: Set[int] = set()
    absorbed: Set[int] = set()
    for r2 in sorted(i for i in members if graph.ops[i].op in ("row_mean", "row_sum")):
        mv = graph.ops[r2].op == "row_mean"
        t1 = graph.ops[r2].inputs[0]
        j = made.get(t1)
        if j is None or graph.ops[j].op != ("square" if mv else "exp"):
            continue
        t2 = graph.ops[j].inputs[0]
        k = made.get(t2)
        if k is None or graph.ops[k].op != "sub":
            continue
        x, m = graph.ops[k].inputs
        r1 = made.get(m)
        if r1 is None or graph.ops[r1].op != ("row_mean" if mv else "row_max") or graph.ops[r1].inputs[0] != x:
            continue
        if readers.get(t1, 0) != 1 or readers.get(t2, 0) != 1:
            continue
        if graph.tensors[t1].role == "out" or graph.tensors[t2].role == "out":
            continue
        if r1 in taken or r1 in first_of:
            continue
        first_of[r2] = r1
        taken.add(r1)
        absorbed.update((j, k))
    return first_of, absorbed


def layout(graph, members: Set[int]):
    """The executor's layout of an op set, or None when it cannot run it:
    {"stages": n, "row_slots": LDS per-row operands, "col_slots": LDS
    per-column operands, "slots": tensors in memory}."""
    fold, members = folded(graph, members)
    ms = sorted(members)
    if not gathers_ok(graph, members, fold):
        return None
    produced = {graph.ops[i].output: i for i in ms}
    touched = set()
    for i in ms:
        if not is_gather(graph.ops[i]):   # a gather's input is addressed, not broadcast
            touched.update(graph.ops[i].inputs)
        touched.add(graph.ops[i].output)
    shape = {t: norm_shape(graph.tensors[t].shape) for t in touched}
    R = C = 1
    for t in touched:
        r, c = shape[t]
        if r != 1:
            R = r
        if c != 1:
            C = c
    for t in touched:
        r, c = shape[t]
        if r not in (1, R) or c not in (1, C):
            return None
    reds = [i for i in ms if graph.ops[i].op in REDUCES]
    if any(shape[graph.ops[i].inputs[0]] != (R, C) for i in reds):
        return None
    # a transpose or a join of full-domain values addresses rows and columns
    gathers2d = any(is_gather(graph.ops[i]) and graph.ops[i].op != "reshape" for i in ms)
    flat = not reds and not gathers2d and all(shape[t] == (R, C) for t in touched)

    def cls(t):
        r, c = shape[t]
        if flat or (r, c) == (R, C):
            return "E"
        if r == 1 and c == C:
            return "COL"
        return "ROW"

    def op_cls(i):
        return "E" if graph.ops[i].op in REDUCES else cls(graph.ops[i].output)
    # tensors in memory: inputs from outside, values needed outside
    outside = set()
    for j, o in enumerate(graph.ops):
        if j not in members:
            outside.update(t for t in o.inputs if t in produced)
    ext = {fold[t][0] if t in fold else t for i in ms for t in graph.ops[i].inputs if t not in produced}
    for i in ms:   # a join of column values would stage two slots in the column phase
        o = graph.ops[i]
        if is_join(o) and cls(o.output) == "ROW":
            return None
    ext |= {t for t in produced if graph.tensors[t].role == "out" or t in outside}
    if len(ext) > MAX_SLOTS:
        return None
    first_of, absorbed = pairs(graph, members)
    avail: Dict[int, int] = {}
    stage: Dict[int, int] = {}
    for i in ms:
        o = graph.ops[i]
        if i in absorbed:
            continue
        if i in first_of:
            st = stage[first_of[i]]   # the first reduction's pass
        else:
            st = max([avail[t] for t in o.inputs if t in produced and t in avail], default=0)
        if op_cls(i) == "COL" and st > 0:
            return None
        stage[i] = st
        avail[o.output] = st + 1 if o.op in REDUCES else st
    for r in reds:
        out = graph.ops[r].output
        if any(out in graph.ops[i].inputs for i in ms) and cls(out) != "ROW":
            return None
    n_stages = max(stage.values()) + 1
    if n_stages > MAX_STAGES:
        return None
    singles = [r for r in reds if r not in first_of]
    if len({stage[r] for r in singles}) != len(singles):
        return None
    row_lds, col_lds = set(), set()
    for i in ms:
        o = graph.ops[i]
        c = op_cls(i)
        if is_gather(o) or i in absorbed:
            continue
        for t in o.inputs:
            if c == "E":
                if cls(t) == "ROW":
                    row_lds.add(t)
                elif cls(t) == "COL":
                    col_lds.add(t)
            elif c == "ROW" and t in produced:
                j = produced[t]
                if graph.ops[j].op in REDUCES or stage[j] != stage[i]:
                    row_lds.add(t)
    if len(row_lds) > MAX_LDS_ROW or len(col_lds) > MAX_LDS_COL:
        return None
    for i in ms:
        c = op_cls(i)
        if c == "E" or is_gather(graph.ops[i]):
            continue
        for t in graph.ops[i].inputs:
            if cls(t) == c:
                continue
            if c == "COL" and t not in produced and shape[t] == (1, 1):
                continue
            return None
    return {"stages": n_stages, "row_slots": len(row_lds), "col_slots": len(col_lds),
            "slots": len(ext)}


def group_ok(graph, members: Set[int]) -> bool:
    """Whether the executor runs this op set as one launch (module
    docstring)."""
    return layout(graph, members) is not None


def partition(graph, fuse: bool = True, row_resident: bool = False):
    """The oracle's grouping with every merge also runnable by the
    executor: the grouping the library must make."""
    return pt.partition(graph, fuse=fuse, row_resident=row_resident, feasible=group_ok)
