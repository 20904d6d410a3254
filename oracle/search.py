"""DisCo's backtracking search over fusion plans, on one GPU (oracle: test
infrastructure only; nothing in the product path imports it).

Follows DisCo (arXiv 2209.12769), "Strategy Maker" (the search of its
Sec. 4.5) in the page's order:

* The strategy space for computation ops (Sec. 3.2 (i), (ii)): fuse an op
  with one of its predecessors, by non-duplicate or by duplicate fusion.
  Method (iii), combining AllReduce instructions, has nothing to act on
  with one GPU and no AllReduce; it is not applied.
* A priority queue Q of candidate plans ordered by Cost holds, at first,
  the original program: every op its own launch.
* Each step dequeues the cheapest plan H.  Each method in turn is applied
  to H n times (RandomApply), n drawn from 0..beta, and its result H' is
  costed once; so each step makes one candidate per method, and the
  candidates of later steps mix the methods.  H' becomes the best plan
  when it is cheaper than the best so far; it is enqueued when its cost is
  at most alpha times the best cost (after that update).
* The search ends when Q is empty or the best plan has not changed for
  max_stall steps (1000 on the page), or after max_steps steps when given.

The cost is a function the caller passes in: on the GPU the measured time
of each group's launch (the page's simulator and GNN are replaced by
measurement); in the tests a byte count.

Readings where the page is silent (the body of its Alg. 1 is not in the
text):
* "Fuse op v with a predecessor p" merges the group holding p into the
  group holding v (ops of the current module may already be fused).  v is
  drawn uniformly over the ops that have a predecessor op in another
  group, p uniformly over v's predecessor ops in other groups (both in
  program order).  Nothing happens when no op has one.
* Duplicate fusion, when p has more than one reader: a copy of p, placed
  right before v and read by v instead of p, joins v's group; p stays
  where it is for its other readers.  With a single reader it is the same
  merge as non-duplicate fusion.
* A move whose result is not a valid plan is not applied (the page's
  validity check, made per move): the group graph must stay acyclic and
  every group within the op and argument limits and runnable by the
  executor (group_ok).
* Random numbers come from SplitMix64 (Steele, Lea and Flood, "Fast
  splittable pseudorandom number generators", OOPSLA 2014), seeded by the
  caller; below(n) is the next output modulo n.  Draw order: per step,
  for each method, its n, then per application v and then p.
* One candidate per method and step: with a single candidate per step
  the queue would never hold more than one plan, and the backtracking the
  page describes would not happen.
* A candidate equal to one enqueued before (the same program and the same
  grouping) is not enqueued again; with a deterministic cost, plateaus of
  equal plans would otherwise fill the queue and starve the rest of it.
* Ties in Q are broken by insertion order.
"""
from __future__ import annotations

import heapq
from typing import Callable, Dict, List, Set, Tuple

from oracle import partition as pt
from oracle.evaluate import norm_shape

MASK64 = (1 << 64) - 1


class SplitMix64:
    """The generator of Steele, Lea and Flood (2014): a Weyl sequence with
    increment 0x9E3779B97F4A7C15, each state mixed by two xor-shift-multiply
    rounds and a final xor-shift."""

    def __init__(self, seed: int):
        self.state = seed & MASK64

    def next(self) -> int:
        self.state = (self.state + 0x9E3779B97F4A7C15) & MASK64
        z = self.state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
        return z ^ (z >> 31)

    def below(self, n: int) -> int:
        return self.next() % n


# ---------------------------------------------------------------- validity
def group_ok(graph, members: Set[int]) -> bool:
    """Whether the executor runs this op set as one launch, from the shapes
    and the dataflow alone: one broadcast domain [R,C]; reductions over it;
    a reduction's result read in the group only by later stages, as a
    per-row value, at most four stages and one reduction each; column ops
    before any reduction; row and column ops reading their own kind (a
    column op may also read a [1,1] input); at most 16 tensors in memory,
    8 per-row and 4 per-column operands held on chip."""
    ms = sorted(members)
    if not pt.gathers_ok(graph, members):
        return False
    produced = {graph.ops[i].output: i for i in ms}
    touched = set()
    for i in ms:
        if graph.ops[i].op not in pt.GATHERS:   # a gather's input is addressed, not broadcast
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
            return False
    reds = [i for i in ms if graph.ops[i].op in pt._REDUCES]
    if any(shape[graph.ops[i].inputs[0]] != (R, C) for i in reds):
        return False
    # a transpose or concat of a full-domain value addresses rows and columns
    gathers2d = any(graph.ops[i].op in ("transpose", "concat") for i in ms)
    flat = not reds and not gathers2d and all(shape[t] == (R, C) for t in touched)

    def cls(t):
        r, c = shape[t]
        if flat or (r, c) == (R, C):
            return "E"
        if r == 1 and c == C:
            return "COL"
        return "ROW"

    def op_cls(i):
        return "E" if graph.ops[i].op in pt._REDUCES else cls(graph.ops[i].output)
    # tensors in memory: inputs from outside, values needed outside
    outside = set()
    for j, o in enumerate(graph.ops):
        if j not in members:
            outside.update(t for t in o.inputs if t in produced)
    ext = {t for i in ms for t in graph.ops[i].inputs if t not in produced}
    for i in ms:   # a concat of column values stages two slots in the column phase
        o = graph.ops[i]
        if o.op == "concat" and cls(o.output) == "ROW":
            return False
    ext |= {t for t in produced if graph.tensors[t].role == "out" or t in outside}
    if len(ext) > pt.MAX_GROUP_ARGS:
        return False
    avail: Dict[int, int] = {}
    stage: Dict[int, int] = {}
    for i in ms:
        o = graph.ops[i]
        st = max([avail[t] for t in o.inputs if t in produced], default=0)
        if op_cls(i) == "COL" and st > 0:
            return False
        stage[i] = st
        avail[o.output] = st + 1 if o.op in pt._REDUCES else st
    for r in reds:
        out = graph.ops[r].output
        if any(out in graph.ops[i].inputs for i in ms) and cls(out) != "ROW":
            return False
    if max(stage.values()) + 1 > pt.MAX_STAGES:
        return False
    if len({stage[r] for r in reds}) != len(reds):
        return False
    row_lds, col_lds = set(), set()
    for i in ms:
        o = graph.ops[i]
        c = op_cls(i)
        if o.op in pt.GATHERS:
            continue
        for t in o.inputs:
            if c == "E":
                if cls(t) == "ROW":
                    row_lds.add(t)
                elif cls(t) == "COL":
                    col_lds.add(t)
            elif c == "ROW" and t in produced:
                j = produced[t]
                if graph.ops[j].op in pt._REDUCES or stage[j] != stage[i]:
                    row_lds.add(t)
    if len(row_lds) > 8 or len(col_lds) > 4:
        return False
    for i in ms:
        c = op_cls(i)
        if c == "E" or graph.ops[i].op in pt.GATHERS:
            continue
        for t in graph.ops[i].inputs:
            if cls(t) == c:
                continue
            if c == "COL" and t not in produced and shape[t] == (1, 1):
                continue
            return False
    return True


def groups_of(labels: List[int]) -> List[List[int]]:
    by: Dict[int, List[int]] = {}
    for i, lab in enumerate(labels):
        by.setdefault(lab, []).append(i)
    return list(by.values())


def plan_ok(graph, labels: List[int]) -> bool:
    """A valid plan: the group graph is acyclic (so every group is convex)
    and every group is within the limits and runnable (group_ok)."""
    groups = groups_of(labels)
    for g in groups:
        if len(g) > pt.MAX_FUSED_OPS or not group_ok(graph, set(g)):
            return False
    owner = {graph.ops[i].output: labels[i] for i in range(len(graph.ops))}
    succ: Dict[int, Set[int]] = {lab: set() for lab in set(labels)}
    for j, o in enumerate(graph.ops):
        for t in o.inputs:
            if t in owner and owner[t] != labels[j]:
                succ[owner[t]].add(labels[j])
    indeg = {lab: 0 for lab in succ}
    for a in succ:
        for b in succ[a]:
            indeg[b] += 1
    ready = [lab for lab in indeg if indeg[lab] == 0]
    seen = 0
    while ready:
        a = ready.pop()
        seen += 1
        for b in succ[a]:
            indeg[b] -= 1
            if indeg[b] == 0:
                ready.append(b)
    return seen == len(succ)


# ---------------------------------------------------------------- moves
def _predecessors(graph, v: int) -> List[int]:
    prod = {o.output: i for i, o in enumerate(graph.ops)}
    return sorted({prod[t] for t in graph.ops[v].inputs if t in prod})


def _readers(graph, t: int) -> List[int]:
    return [j for j, o in enumerate(graph.ops) if t in o.inputs]


def _with_copy(graph, origin, labels, p: int, v: int):
    """Copy op p right before v; v reads the copy, which joins v's group."""
    from workloads.graph import Graph, OpDesc, TensorDesc
    op = graph.ops[p]
    d = graph.tensors[op.output]
    tensors = list(graph.tensors) + [TensorDesc(f"{d.name}@{len(graph.tensors)}", d.dtype, d.shape, "tmp")]
    nt = len(tensors) - 1
    o = graph.ops[v]
    ops = (list(graph.ops[:v]) + [OpDesc(op.op, op.inputs, nt, op.imm, op.opaque)]
           + [OpDesc(o.op, tuple(nt if t == op.output else t for t in o.inputs), o.output, o.imm,
                     o.opaque)] + list(graph.ops[v + 1:]))
    return (Graph(tensors, ops), origin[:v] + [origin[p]] + origin[v:],
            labels[:v] + [labels[v]] + labels[v:])


def fuse_move(state, rng: SplitMix64, duplicate: bool):
    """One application of method (i) (duplicate False) or (ii) (True)."""
    graph, origin, labels = state
    cross = [[p for p in _predecessors(graph, v) if labels[p] != labels[v]]
             for v in range(len(graph.ops))]
    eligible = [v for v in range(len(graph.ops)) if cross[v]]
    if not eligible:
        return state
    v = eligible[rng.below(len(eligible))]
    p = cross[v][rng.below(len(cross[v]))]
    if duplicate and len(_readers(graph, graph.ops[p].output)) > 1:
        cand = _with_copy(graph, origin, labels, p, v)
    else:
        lp, lv = labels[p], labels[v]
        cand = (graph, origin, [lv if x == lp else x for x in labels])
    return cand if plan_ok(cand[0], cand[2]) else state


def state_key(state):
    """A plan's identity: its program and its grouping, labels renumbered
    in order of first appearance."""
    graph, _, labels = state
    ren: Dict[int, int] = {}
    lab = tuple(ren.setdefault(x, len(ren)) for x in labels)
    ops = tuple((o.op, o.inputs, o.output, o.imm, o.opaque) for o in graph.ops)
    return ops, lab


def search(graph, cost: Callable, alpha: float = 1.05, beta: int = 10, max_stall: int = 1000,
           seed: int = 0, max_steps: int = 0):
    """Returns ((program, origin, labels) of the best plan, stats).  cost is
    called as cost(program, groups) with groups as lists of op indices."""
    rng = SplitMix64(seed)
    n = len(graph.ops)
    start = (graph, list(range(n)), list(range(n)))
    c0 = float(cost(graph, groups_of(start[2])))
    queue: List[Tuple[float, int, tuple]] = [(c0, 0, start)]
    seen = {state_key(start)}
    best, c_best = start, c0
    stall = steps = evals = 0
    tick = 1
    while queue and stall < max_stall and (max_steps == 0 or steps < max_steps):
        _, _, h = heapq.heappop(queue)
        steps += 1
        improved = False
        for dup in (False, True):
            cand = h
            for _ in range(rng.below(beta + 1)):
                cand = fuse_move(cand, rng, dup)
            cc = float(cost(cand[0], groups_of(cand[2])))
            evals += 1
            if cc < c_best:
                best, c_best, improved = cand, cc, True
            key = state_key(cand)
            if cc <= alpha * c_best and key not in seen:
                seen.add(key)
                heapq.heappush(queue, (cc, tick, cand))
                tick += 1
        stall = 0 if improved else stall + 1
    return best, {"steps": steps, "evaluations": evals, "start_cost": c0, "best_cost": c_best,
                  "queue_left": len(queue)}


def bytes_cost(graph, groups) -> float:
    """A deterministic cost for tests: HBM bytes plus 65536 per launch."""
    b, launches = pt.plan_cost(graph, groups)
    return float(b + 65536 * launches)
