"""Pattern annotation, post-dominators and the grouping rule (oracle, test
infrastructure only).

Follows Apache TVM, "Operator Fusion" (docs/arch/fusion.rst), in its order:

1. Annotate (section "Operator Pattern Classification", the OpPatternKind
   table): kElemWise 0 when every operand has the result's shape,
   kBroadcast 1 when some operand is broadcast, kInjective 2 for copy
   and the moves, kCommReduce 3 for the row reductions, kTuple 7 for a
   tuple, kOpaque 8 when forced.  A group's pattern is the max over its
   members (CombinePattern), a tuple that has fused into a later group
   counting as kInjective there (the table: a tuple fuses into the
   injective ops after it).
2. Forward graph (section "Algorithm", step 1): one node per op, an edge
   from an op to every op that reads its output.
3. Post-dominators (step 2): here from their definition, not from the LCA
   construction the page describes.  A virtual exit follows every node
   whose output is a graph output or has no reader; pdom(exit) = {exit} and
   pdom(n) = {n} u (intersection of pdom(s) over n's successors s).  The
   immediate post-dominator is the strict post-dominator nearest to n.
4. Fuse (step 3 and "Fusion rules"): three phases; in each, nodes in
   topological order.  A node is skipped when it already shares a group
   with its immediate post-dominator d, or has none.  Its group's pattern
   picks the rule:
     <= kBroadcast : every node strictly between n and d on any path is
                     <= kInjective, and d's group is <= kCommReduce;
     kInjective, kTuple : (phase 1 and later) everything on the paths and
                     d's group are <= kInjective;
     kCommReduce   : never initiates (reductions are sinks only);
     kOpaque       : never fuses (a barrier).
   A post-dominator that is a tuple takes fields only by phase 2's rule:
   in phase 2, a node <= kInjective whose d is a tuple that has already
   fused into a later group (its group's root is no longer the tuple)
   fuses when every node on the paths is <= kInjective.
   Limits: at most 256 ops per group (kMaxFusedOps) and at most
   MAX_GROUP_ARGS external tensors per group (the page names an argument
   limit without its value; 16 is the reading taken here).  CommitFuse puts
   n, d and every node on a path between them into one group (union-find).

Readings where the page is silent: the source's pattern is its group's
pattern; path nodes are judged by their own pattern; a node whose output
is a graph output has no post-dominator.

Injective ops that move elements (transpose, reshape, concat; kInjective
in the page's table) fuse by the same phases.  A tuple (kTuple) holds two
fields; its only reader is a concat of that tuple alone.

Row-resident extension (opt-in, row_resident=True; beyond the page, whose
fusion rules keep a reduction as the last op of its group): after the
three phases, a group holding a row reduction r is merged with the group of
an op c (not opaque) that reads r's result, scanning r then c in ascending
order and starting over after every merge, when
  * the merge is convex: no op outside the two groups lies on a path from
    one to the other (the group graph stays acyclic);
  * the merged set keeps the op and argument limits.

What runs a group may hold less than these rules allow (one kernel launch
has finite registers, LDS and stages).  `feasible(graph, members)`, when
given, is one more condition on every merge of the phases and of the
row-resident pass; the oracle's own rules are those above and no more.

Duplicate fusion (opt-in, duplicate(); DisCo, "Background and Motivation"
on the two fusion approaches for a predecessor with several successors,
and "Strategy Maker", method (ii): duplicate the predecessor for its other
successors).  The page leaves the choice to its search; the rule here
decides it by the bytes it moves, the reason the page gives for
duplicating.  Before grouping, ops are scanned in program order.  For an
elementwise or broadcast op p with two or more readers, some of which are
in another group than p (and not opaque):
  * each such reader r gets its own copy of p, placed right before r and
    writing a new intermediate that r reads instead of p's output;
  * p itself is dropped when its output is an intermediate that no op
    reads any more.
The rewrite is kept when every reader of every copy (this rewrite's and
earlier ones') then shares the copy's group, so no copy's value is ever
stored, and the plan's cost (HBM bytes, then launches; plan_cost) strictly
drops; the scan then starts over.  Otherwise p is not tried again.

Pinned in tests/test_oracle_partition.py: the page's add/exp/squeeze example
and its diamond, the sink-only and barrier rules, the 256 limit, and the
post-dominator sets against path enumeration on every small DAG.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Set

from .evaluate import norm_shape

K_ELEMWISE, K_BROADCAST, K_INJECTIVE, K_COMM_REDUCE = 0, 1, 2, 3
K_OUT_EWISE_FUSABLE, K_TUPLE, K_OPAQUE = 4, 7, 8

# injective ops that move elements to other positions (the page's table
# makes transpose, reshape and concatenate injective)
MOVES = ("transpose", "reshape", "concat")

MAX_FUSED_OPS = 256
MAX_GROUP_ARGS = 16
_REDUCES = ("row_sum", "row_mean", "row_max")


def pattern(graph, i: int) -> int:
    o = graph.ops[i]
    if o.opaque:
        return K_OPAQUE
    if o.op in _REDUCES:
        return K_COMM_REDUCE
    if o.op == "tuple":
        return K_TUPLE
    if o.op in ("copy",) + MOVES:
        return K_INJECTIVE
    out = norm_shape(graph.tensors[o.output].shape)
    if any(norm_shape(graph.tensors[t].shape) != out for t in o.inputs):
        return K_BROADCAST
    return K_ELEMWISE


def successors(graph) -> List[List[int]]:
    readers: Dict[int, List[int]] = {}
    for j, o in enumerate(graph.ops):
        for t in set(o.inputs):
            readers.setdefault(t, []).append(j)
    succ = []
    for i, o in enumerate(graph.ops):
        succ.append(sorted(set(readers.get(o.output, []))))
    return succ


def exits_to_end(graph, i: int, succ) -> bool:
    o = graph.ops[i]
    return graph.tensors[o.output].role == "out" or not succ[i]


def postdominator_sets(graph) -> List[Set[int]]:
    """pdom(n) as sets of op indices; -1 stands for the virtual exit."""
    n = len(graph.ops)
    succ = successors(graph)
    pd: List[Optional[Set[int]]] = [None] * n
    for i in range(n - 1, -1, -1):           # readers come later in the order
        sets = [pd[s] for s in succ[i]]
        if exits_to_end(graph, i, succ):
            sets.append({-1})
        common = set.intersection(*sets)
        pd[i] = {i} | common
    return pd  # type: ignore[return-value]


def immediate_postdominators(graph) -> List[Optional[int]]:
    pd = postdominator_sets(graph)
    ipd: List[Optional[int]] = []
    for i, s in enumerate(pd):
        strict = s - {i}
        if strict == {-1}:
            ipd.append(None)
            continue
        # the nearest strict post-dominator is the one every other strict
        # post-dominator of n also post-dominates
        cand = [d for d in strict if d != -1 and strict - {d} <= pd[d]]
        assert len(cand) == 1, (i, strict)
        ipd.append(cand[0])
    return ipd


def _reach(succ, start: int) -> Set[int]:
    seen, stack = set(), [start]
    while stack:
        v = stack.pop()
        for s in succ[v]:
            if s not in seen:
                seen.add(s)
                stack.append(s)
    return seen


def _between(succ, pred, a: int, b: int) -> Set[int]:
    """Nodes strictly between a and b on some path a -> b."""
    fwd = _reach(succ, a)
    back = _reach(pred, b)
    return (fwd & back) - {a, b}


class _UnionFind:
    def __init__(self, n: int, pats: List[int]):
        self.parent = list(range(n))
        self.pat = list(pats)
        self.size = [1] * n

    def find(self, x: int) -> int:
        while self.parent[x] != x:
            x = self.parent[x]
        return x

    def union_into(self, x: int, root_target: int) -> None:
        rx, rt = self.find(x), self.find(root_target)
        if rx == rt:
            return
        self.parent[rx] = rt
        # a tuple fused into the group after it is an injective member there
        self.pat[rt] = max(self.pat[rt], K_INJECTIVE if self.pat[rx] == K_TUPLE else self.pat[rx])
        self.size[rt] += self.size[rx]


def _group_args(graph, members: Set[int]) -> int:
    produced = {graph.ops[i].output for i in members}
    ext = set()
    for i in members:
        for t in graph.ops[i].inputs:
            if t not in produced:
                ext.add(t)
    for j, o in enumerate(graph.ops):
        if j in members:
            continue
        for t in o.inputs:
            if t in produced:
                ext.add(t)
    for t in produced:
        if graph.tensors[t].role == "out":
            ext.add(t)
    return len(ext)


def _convex(succ, members: Set[int]) -> bool:
    """No path leaves the set and comes back into it."""
    outside = {s for v in members for s in succ[v] if s not in members}
    seen, stack = set(), list(outside)
    while stack:
        v = stack.pop()
        if v in seen:
            continue
        seen.add(v)
        for s in succ[v]:
            if s in members:
                return False
            stack.append(s)
    return True


def partition(graph, fuse: bool = True, row_resident: bool = False,
              feasible=None) -> List[List[int]]:
    """Groups of op indices, each sorted, listed in an order that respects
    the dependencies between groups.  feasible(graph, members), when given,
    must also hold for every merge (module docstring)."""
    n = len(graph.ops)
    pats = [pattern(graph, i) for i in range(n)]
    uf = _UnionFind(n, pats)
    if fuse and n:
        succ = successors(graph)
        pred: List[List[int]] = [[] for _ in range(n)]
        for i, ss in enumerate(succ):
            for s in ss:
                pred[s].append(i)
        ipd = immediate_postdominators(graph)
        for phase in range(3):
            for i in range(n):
                d = ipd[i]
                if d is None or uf.find(i) == uf.find(d):
                    continue
                src_pat = uf.pat[uf.find(i)]
                sink_pat = uf.pat[uf.find(d)]
                mid = _between(succ, pred, i, d)
                if graph.ops[d].op == "tuple":
                    # phase 2: into a tuple already fused into a later group
                    ok = (phase == 2 and src_pat <= K_INJECTIVE and uf.find(d) != d
                          and all(pats[m] <= K_INJECTIVE for m in mid))
                elif src_pat <= K_BROADCAST:
                    ok = (all(pats[m] <= K_INJECTIVE for m in mid)
                          and sink_pat <= K_COMM_REDUCE)
                elif src_pat in (K_INJECTIVE, K_TUPLE) and phase >= 1:
                    ok = (all(pats[m] <= K_INJECTIVE for m in mid)
                          and sink_pat <= K_INJECTIVE)
                else:
                    ok = False
                if not ok:
                    continue
                roots = {uf.find(v) for v in mid | {i, d}}
                members = {v for v in range(n) if uf.find(v) in roots}
                if len(members) > MAX_FUSED_OPS:
                    continue
                if _group_args(graph, members) > MAX_GROUP_ARGS:
                    continue
                if feasible is not None and not feasible(graph, members):
                    continue
                for v in mid | {i}:
                    uf.union_into(v, d)
        if row_resident:
            changed = True
            while changed:
                changed = False
                for r in range(n):
                    if changed or graph.ops[r].op not in _REDUCES:
                        continue
                    out = graph.ops[r].output
                    for c in range(n):
                        if out not in graph.ops[c].inputs or uf.find(c) == uf.find(r):
                            continue
                        if pats[c] == K_OPAQUE:
                            continue
                        roots = {uf.find(r), uf.find(c)}
                        members = {v for v in range(n) if uf.find(v) in roots}
                        if not _convex(succ, members):
                            continue
                        if len(members) > MAX_FUSED_OPS or _group_args(graph, members) > MAX_GROUP_ARGS:
                            continue
                        if feasible is not None and not feasible(graph, members):
                            continue
                        uf.union_into(r, c)
                        changed = True
                        break
    groups: Dict[int, List[int]] = {}
    for i in range(n):
        groups.setdefault(uf.find(i), []).append(i)
    return _order_groups(graph, list(groups.values()))


def _order_groups(graph, groups: List[List[int]]) -> List[List[int]]:
    owner = {}
    for gi, g in enumerate(groups):
        for i in g:
            owner[graph.ops[i].output] = gi
    deps = [set() for _ in groups]
    for gi, g in enumerate(groups):
        for i in g:
            for t in graph.ops[i].inputs:
                if t in owner and owner[t] != gi:
                    deps[gi].add(owner[t])
    order, done = [], set()
    while len(order) < len(groups):
        ready = [gi for gi in range(len(groups)) if gi not in done and deps[gi] <= done]
        if not ready:
            raise ValueError("groups depend on each other in a cycle")
        gi = min(ready, key=lambda k: min(groups[k]))
        order.append(gi)
        done.add(gi)
    return [sorted(groups[gi]) for gi in order]


def stored_tensors(graph, groups: List[List[int]]) -> Set[int]:
    """Intermediates written to memory: read by an op of another group."""
    owner = {}
    for gi, g in enumerate(groups):
        for i in g:
            owner[graph.ops[i].output] = gi
    stored = set()
    for gi, g in enumerate(groups):
        for i in g:
            for t in graph.ops[i].inputs:
                if t in owner and owner[t] != gi:
                    stored.add(t)
    return stored


_DT_BYTES = {"f32": 4, "bf16": 2, "u8": 1}


def _tensor_bytes(graph, t: int) -> int:
    d = graph.tensors[t]
    n = 1
    for e in d.shape:
        n *= e
    return n * _DT_BYTES[d.dtype]


def plan_cost(graph, groups: List[List[int]]):
    """(HBM bytes, launches) of a grouping: per group, every distinct tensor
    it reads from memory (graph inputs and values stored by other groups)
    and every tensor it stores (graph outputs and values other groups
    read)."""
    owner = {}
    for gi, g in enumerate(groups):
        for i in g:
            owner[graph.ops[i].output] = gi
    stored = stored_tensors(graph, groups) | set(graph.outputs())
    total = 0
    for gi, g in enumerate(groups):
        touched = set()
        for i in g:
            for t in graph.ops[i].inputs:
                if owner.get(t) != gi:
                    touched.add(t)
            if graph.ops[i].output in stored:
                touched.add(graph.ops[i].output)
        total += sum(_tensor_bytes(graph, t) for t in touched)
    return total, len(groups)


def _duplicate_op(graph, origin: List[int], p: int, targets: List[int]):
    """The program with op p copied for each reader in targets (see the
    module docstring); returns (graph, origin, copy op ids)."""
    from workloads.graph import Graph, OpDesc, TensorDesc
    op = graph.ops[p]
    tensors = list(graph.tensors)
    new_t = {}
    for r in targets:
        d = graph.tensors[op.output]
        tensors.append(TensorDesc(f"{d.name}@{r}", d.dtype, d.shape, "tmp"))
        new_t[r] = len(tensors) - 1
    still_read = any(op.output in graph.ops[j].inputs
                     for j in range(len(graph.ops)) if j not in new_t)
    drop = not still_read and graph.tensors[op.output].role == "tmp"
    ops, org, copies = [], [], []
    for j, o in enumerate(graph.ops):
        if j in new_t:
            copies.append(len(ops))
            ops.append(OpDesc(op.op, op.inputs, new_t[j], op.imm, op.opaque))
            org.append(origin[p])
            ins = tuple(new_t[j] if t == op.output else t for t in o.inputs)
            ops.append(OpDesc(o.op, ins, o.output, o.imm, o.opaque))
            org.append(origin[j])
        elif not (j == p and drop):
            ops.append(o)
            org.append(origin[j])
    return Graph(tensors, ops), org, copies


def duplicate(graph, row_resident: bool = False, feasible=None):
    """Duplicate fusion (module docstring).  Returns (program, origin):
    the rewritten graph, whose tensors extend the input graph's, and for
    each of its ops the op of the input graph it computes.  feasible is
    passed to every partition made on the way."""
    g, origin = graph, list(range(len(graph.ops)))
    blocked: Set[int] = set()
    while True:
        groups = partition(g, row_resident=row_resident, feasible=feasible)
        cost = plan_cost(g, groups)
        gof = {i: k for k, grp in enumerate(groups) for i in grp}
        kept = False
        for p in range(len(g.ops)):
            if origin[p] in blocked or pattern(g, p) > K_BROADCAST:
                continue
            out = g.ops[p].output
            readers = [r for r in range(len(g.ops)) if out in g.ops[r].inputs]
            if len(readers) < 2:
                continue
            targets = [r for r in readers if gof[r] != gof[p] and pattern(g, r) != K_OPAQUE]
            if not targets:
                continue
            g2, org2, copies = _duplicate_op(g, origin, p, targets)
            groups2 = partition(g2, row_resident=row_resident, feasible=feasible)
            gof2 = {i: k for k, grp in enumerate(groups2) for i in grp}
            # no value of a copy (this rewrite's or an earlier one's) is
            # stored: every reader of a copy shares the copy's group
            fused = all(gof2[j] == gof2[i]
                        for i, o in enumerate(g2.ops) if o.output >= len(graph.tensors)
                        for j, q in enumerate(g2.ops) if o.output in q.inputs)
            if fused and plan_cost(g2, groups2) < cost:
                g, origin, kept = g2, org2, True
                break
            blocked.add(origin[p])
        if not kept:
            return g, origin
