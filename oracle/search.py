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
  validity check, made per move).  Valid (plan_ok): the group graph is
  acyclic, no opaque op (the page's parameter and control-flow ops, which
  are never fused) shares a group, and every group keeps TVM's op and
  argument limits.  What runs the plan may hold less: feasible(graph,
  members), when the caller gives one, must hold for every group too.
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
def groups_of(labels: List[int]) -> List[List[int]]:
    by: Dict[int, List[int]] = {}
    for i, lab in enumerate(labels):
        by.setdefault(lab, []).append(i)
    return list(by.values())


def _args(graph, members: Set[int]) -> int:
    """Tensors a group touches in memory: inputs made outside it, and its
    values read outside it or returned by the graph."""
    produced = {graph.ops[i].output for i in members}
    ext = {t for i in members for t in graph.ops[i].inputs if t not in produced}
    for j, o in enumerate(graph.ops):
        if j not in members:
            ext.update(t for t in o.inputs if t in produced)
    ext.update(t for t in produced if graph.tensors[t].role == "out")
    return len(ext)


def plan_ok(graph, labels: List[int], feasible=None) -> bool:
    """A valid plan (module docstring): the group graph is acyclic (so
    every group is convex), no opaque op is fused, every group keeps the op
    and argument limits, and feasible(graph, members) holds when given."""
    groups = groups_of(labels)
    for g in groups:
        if len(g) > pt.MAX_FUSED_OPS or _args(graph, set(g)) > pt.MAX_GROUP_ARGS:
            return False
        if len(g) > 1 and any(pt.pattern(graph, i) == pt.K_OPAQUE for i in g):
            return False
        if feasible is not None and not feasible(graph, set(g)):
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


def fuse_move(state, rng: SplitMix64, duplicate: bool, feasible=None):
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
    return cand if plan_ok(cand[0], cand[2], feasible) else state


def state_key(state):
    """A plan's identity: its program and its grouping, labels renumbered
    in order of first appearance."""
    graph, _, labels = state
    ren: Dict[int, int] = {}
    lab = tuple(ren.setdefault(x, len(ren)) for x in labels)
    ops = tuple((o.op, o.inputs, o.output, o.imm, o.opaque) for o in graph.ops)
    return ops, lab


def search(graph, cost: Callable, alpha: float = 1.05, beta: int = 10, max_stall: int = 1000,
           seed: int = 0, max_steps: int = 0, feasible=None):
    """Returns ((program, origin, labels) of the best plan, stats).  cost is
    called as cost(program, groups) with groups as lists of op indices;
    feasible, when given, bounds every group of every plan (plan_ok)."""
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
                cand = fuse_move(cand, rng, dup, feasible)
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
