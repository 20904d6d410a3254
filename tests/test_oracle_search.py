"""Pins for the oracle's backtracking search over fusion plans (DisCo,
"Strategy Maker"): its random source against the generator's published
outputs, the validity rule against the fusion pass's own groupings and a
hand-made cycle, the search against exhaustive enumeration of every
grouping on small graphs, and its queue and stall rules on cases whose
trajectory is known."""
import numpy as np

from oracle import evaluate as oev
from oracle import partition as pt
from oracle import search as sr
from tests.test_oracle_partition import _f32_reduce_dags, _random_dags
from workloads import configs
from workloads.graph import Graph


def test_splitmix64_published_outputs():
    # the first outputs from state 0, as published with the generator's
    # reference implementation, and the widely used seed-1234567 vectors
    r = sr.SplitMix64(0)
    assert [r.next() for _ in range(4)] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4,
                                            0x06C45D188009454F, 0xF88BB8A8724C81EC]
    r = sr.SplitMix64(1234567)
    assert [r.next() for _ in range(3)] == [6457827717110365317, 3203168211198807973,
                                            9817491932198370423]


def _labels(groups, n):
    lab = [0] * n
    for k, g in enumerate(groups):
        for i in g:
            lab[i] = k
    return lab


def test_plan_ok_accepts_the_fusion_pass_groupings():
    graphs = [configs.layernorm_graph(16, 64), configs.c3_graph(8, 64, head_op=True),
              configs.c2_graph(4, 16), configs.gelu_graph(4, 16), configs.dropout_graph(4, 16)]
    graphs += list(_f32_reduce_dags(5, 150))
    for g in graphs:
        for kw in ({}, {"row_resident": True}, {"fuse": False}):
            groups = pt.partition(g, **kw)
            assert sr.plan_ok(g, _labels(groups, len(g.ops))), (kw, groups)


def test_plan_ok_rejects_a_cycle_an_opaque_fusion_and_the_limits():
    # x -> a -> b -> c with {a, c} together and b alone: a path leaves the
    # group and comes back
    g = Graph()
    x = g.input("x", "f32", (4, 8))
    a = g.op("exp", [x], "a", "f32", (4, 8))
    b = g.op("neg", [a], "b", "f32", (4, 8))
    g.op("relu", [b], "c", "f32", (4, 8), role="out")
    assert sr.plan_ok(g, [0, 1, 2]) and sr.plan_ok(g, [0, 0, 0])
    assert not sr.plan_ok(g, [0, 1, 0])
    # an opaque op (the page's parameters and control flow) is never fused
    g = Graph()
    x = g.input("x", "f32", (4, 8))
    a = g.op("exp", [x], "a", "f32", (4, 8))
    g.op("relu", [a], "c", "f32", (4, 8), role="out", opaque=True)
    assert sr.plan_ok(g, [0, 1]) and not sr.plan_ok(g, [0, 0])
    # reduce, then broadcast back, in one group: the pages' rules allow it
    g = Graph()
    x = g.input("x", "f32", (4, 8))
    s = g.op("row_sum", [x], "s", "f32", (4, 1))
    g.op("mul", [x, s], "y", "f32", (4, 8), role="out")
    assert sr.plan_ok(g, [0, 0])
    # the argument limit: 17 inputs summed into one group
    g = Graph()
    xs = [g.input(f"x{k}", "f32", (4, 8)) for k in range(17)]
    acc = g.op("add", [xs[0], xs[1]], "a1", "f32", (4, 8))
    for k in range(2, 17):
        acc = g.op("add", [acc, xs[k]], f"a{k}", "f32", (4, 8), role="out" if k == 16 else "tmp")
    n = len(g.ops)
    assert not sr.plan_ok(g, [0] * n)                  # 17 inputs and the output
    assert sr.plan_ok(g, [0] * 8 + [1] * (n - 8))      # 10 tensors per group


def _set_partitions(items):
    if not items:
        yield []
        return
    first, rest = items[0], items[1:]
    for part in _set_partitions(rest):
        for k in range(len(part)):
            yield part[:k] + [[first] + part[k]] + part[k + 1:]
        yield [[first]] + part


def _connected(g, members):
    """Whether the ops form one piece of the dataflow graph (edges taken
    both ways): the groupings that fusing ops with their predecessors can
    make.  Fusing unrelated ops side by side is not one of DisCo's moves."""
    members = set(members)
    prod = {o.output: i for i, o in enumerate(g.ops)}
    adj = {i: set() for i in members}
    for i in members:
        for t in g.ops[i].inputs:
            j = prod.get(t)
            if j in members:
                adj[i].add(j)
                adj[j].add(i)
    start = min(members)
    seen, stack = {start}, [start]
    while stack:
        for j in adj[stack.pop()]:
            if j not in seen:
                seen.add(j)
                stack.append(j)
    return seen == members


def test_search_finds_the_exhaustive_optimum_on_the_config_graphs():
    """On the configs' small graphs no grouping of the original program
    that fusing ops with predecessors can make (every set partition into
    connected groups that is a valid plan) costs less than what the search
    returns with the page's alpha and beta; on the LayerNorm the search does
    at least as well as the fusion rules."""
    graphs = [configs.c1_graph(4, 16), configs.c2_graph(4, 16), configs.c3_graph(4, 16),
              configs.c3_graph(4, 16, head_op=True), configs.gelu_graph(4, 16),
              configs.dropout_graph(4, 16), configs.layernorm_graph(4, 16)]
    for k, g in enumerate(graphs):
        n = len(g.ops)
        if n <= 7:
            best = min(sr.bytes_cost(g, part) for part in _set_partitions(list(range(n)))
                       if all(_connected(g, grp) for grp in part) and sr.plan_ok(g, _labels(part, n)))
        else:
            # the LayerNorm (11 ops, too many to enumerate): at least as
            # cheap as the fusion rules' three groups
            best = sr.bytes_cost(g, pt.partition(g))
        (prog, origin, lab), stats = sr.search(g, sr.bytes_cost, seed=200 + k)
        assert stats["best_cost"] <= best, (k, stats, best)
        assert sr.plan_ok(prog, lab)


def test_search_result_computes_the_graph():
    """The best plan's program, run group by group, gives the graph's own
    values (all-f32 graphs: stored values round to themselves)."""
    for k, g in enumerate(_f32_reduce_dags(43, 60)):
        (prog, origin, lab), _ = sr.search(g, sr.bytes_cost, seed=k, max_stall=200)
        for i, o in enumerate(prog.ops):
            src = g.ops[origin[i]]
            assert (o.op, o.imm) == (src.op, src.imm)
        ins = {t: configs.tensor_values("f32", g.tensors[t].shape, "uniform", 700 + k, j, -1.5, 1.5)
               for j, t in enumerate(g.inputs())}
        p1 = pt.partition(g)
        _, want = oev.run(g, ins, stored=pt.stored_tensors(g, p1), groups=p1)
        groups = sr.groups_of(lab)
        _, got = oev.run(prog, ins, stored=pt.stored_tensors(prog, groups), groups=groups)
        for t in g.outputs():
            assert np.array_equal(got[t].view(np.uint32), want[t].view(np.uint32))


def test_search_queue_and_stall_rules():
    # one op: nothing can fuse; both candidates are the start plan, which
    # is not enqueued twice, so the queue is empty after one step
    g = Graph()
    x = g.input("x", "f32", (4, 8))
    g.op("exp", [x], "y", "f32", (4, 8), role="out")
    _, st = sr.search(g, sr.bytes_cost, max_stall=37)
    assert st["steps"] == 1 and st["evaluations"] == 2 and st["queue_left"] == 0
    # a chain of 24 ops and a constant cost: no candidate is ever an
    # improvement, new ones keep coming, so only the stall rule ends it
    g = Graph()
    v = g.input("x", "f32", (4, 8))
    for i in range(24):
        v = g.op("neg", [v], f"t{i}", "f32", (4, 8), role="out" if i == 23 else "tmp")
    _, st = sr.search(g, lambda prog, groups: 1.0, beta=3, max_stall=20, seed=9)
    assert st["steps"] == 20 and st["evaluations"] == 40 and st["queue_left"] > 0
    # a cost that grows with every evaluation and alpha = 1: no candidate is
    # enqueued, the queue is empty after one step
    calls = []

    def growing(prog, groups):
        calls.append(1)
        return float(len(calls))
    _, st = sr.search(configs.c2_graph(4, 16), growing, alpha=1.0)
    assert st["steps"] == 1 and st["queue_left"] == 0 and st["best_cost"] == 1.0
    # max_steps bounds the search
    _, st = sr.search(configs.layernorm_shared_graph(4, 8), sr.bytes_cost, max_steps=2)
    assert st["steps"] == 2
    # the same seed gives the same trajectory
    a = sr.search(configs.layernorm_shared_graph(4, 8), sr.bytes_cost, seed=3)
    b = sr.search(configs.layernorm_shared_graph(4, 8), sr.bytes_cost, seed=3)
    assert a[1] == b[1] and a[0][2] == b[0][2] and a[0][1] == b[0][1]
