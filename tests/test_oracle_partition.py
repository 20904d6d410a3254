"""Pins for the oracle's grouping: the page's worked example and diamond, the
sink-only, barrier and size rules, and post-dominators checked against path
enumeration on small DAGs (TVM "Operator Fusion", FuseOps)."""
import itertools
import json
import os

import numpy as np

from oracle import partition as pt
from workloads import configs
from workloads.graph import Graph, OpDesc, TensorDesc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def graph_from_json(d) -> Graph:
    g = Graph()
    for t in d["tensors"]:
        g.tensors.append(TensorDesc(t["name"], t["dtype"], tuple(t["shape"]), t["role"]))
    for o in d["ops"]:
        g.ops.append(OpDesc(o["op"], tuple(o["inputs"]), o["output"], float(o.get("imm", 0.0)),
                            bool(o.get("opaque", False))))
    return g


def as_sets(groups):
    return sorted(sorted(x) for x in groups)


def test_tvm_worked_example_is_one_group():
    with open(os.path.join(GOLDEN, "tvm_add_exp_squeeze.json")) as f:
        d = json.load(f)
    g = graph_from_json(d)
    assert as_sets(pt.partition(g)) == d["expected_groups"]
    assert [pt.pattern(g, i) for i in range(3)] == [pt.K_ELEMWISE, pt.K_ELEMWISE, pt.K_INJECTIVE]


def test_diamond_with_op_head_is_one_group_and_its_ipdom_is_the_join():
    g = configs.c3_graph(8, 64, head_op=True)
    ipd = pt.immediate_postdominators(g)
    assert ipd[0] == 4              # head -> the 3-input add where the branches meet
    assert ipd[1] == ipd[2] == ipd[3] == 4
    assert ipd[4] == 5 and ipd[5] is None
    assert as_sets(pt.partition(g)) == [[0, 1, 2, 3, 4, 5]]


def test_config_groups():
    assert as_sets(pt.partition(configs.c1_graph(4, 8))) == [[0, 1, 2]]
    g2 = configs.c2_graph(4, 8)
    assert as_sets(pt.partition(g2)) == [[0, 1, 2]]
    assert pt.pattern(g2, 0) == pt.K_BROADCAST
    assert as_sets(pt.partition(configs.c3_graph(4, 8))) == [[0, 1, 2, 3, 4]]
    ln = configs.layernorm_graph(4, 8)
    groups = pt.partition(ln)
    # G1 mean; G2 x-mean, square, mean; G3 the normalise chain with rstd hoisted in
    assert as_sets(groups) == [[0], [1, 2, 3], [4, 5, 6, 7, 8, 9, 10]]
    stored = pt.stored_tensors(ln, groups)
    assert {ln.tensors[t].name for t in stored} == {"mean", "var"}
    assert as_sets(pt.partition(configs.gelu_graph(4, 8))) == [[0, 1]]
    assert as_sets(pt.partition(configs.dropout_graph(4, 8))) == [[0, 1]]
    sm = configs.softmax_graph(4, 8)
    # G1 max (a reduction is a sink); G2 x-max, exp, sum; G3 x-max, exp and
    # the product with 1/sum, the reciprocal hoisted in as a row operand
    assert pt.pattern(sm, 0) == pt.K_COMM_REDUCE
    groups = pt.partition(sm)
    assert as_sets(groups) == [[0], [1, 2, 3], [4, 5, 6, 7]]
    assert {sm.tensors[t].name for t in pt.stored_tensors(sm, groups)} == {"max", "sum"}


def test_unfused_mode_is_one_op_per_group():
    ln = configs.layernorm_graph(4, 8)
    assert as_sets(pt.partition(ln, fuse=False)) == [[i] for i in range(11)]


def test_reduction_never_initiates():
    g = Graph()
    x = g.input("x", "f32", (4, 8))
    r = g.op("row_sum", [x], "r", "f32", (4, 1))
    g.op("mul_imm", [r], "y", "f32", (4, 1), role="out", imm=2.0)
    assert as_sets(pt.partition(g)) == [[0], [1]]


def test_opaque_is_a_barrier():
    g = Graph()
    x = g.input("x", "f32", (4, 8))
    a = g.op("exp", [x], "a", "f32", (4, 8))
    b = g.op("neg", [a], "b", "f32", (4, 8), opaque=True)
    g.op("relu", [b], "c", "f32", (4, 8), role="out")
    assert as_sets(pt.partition(g)) == [[0], [1], [2]]
    # an opaque node on one branch of a diamond blocks the whole diamond
    g = Graph()
    x = g.input("x", "f32", (4, 8))
    h = g.op("exp", [x], "h", "f32", (4, 8))
    p = g.op("neg", [h], "p", "f32", (4, 8), opaque=True)
    q = g.op("relu", [h], "q", "f32", (4, 8))
    g.op("add", [p, q], "y", "f32", (4, 8), role="out")
    assert as_sets(pt.partition(g)) == [[0], [1], [2, 3]]


def test_long_chain_splits_at_256_ops():
    g = Graph()
    v = g.input("x", "f32", (2, 8))
    for i in range(300):
        v = g.op("neg", [v], f"t{i}", "f32", (2, 8), role="out" if i == 299 else "tmp")
    sizes = [len(x) for x in pt.partition(g)]
    assert sizes == [256, 44]


def test_argument_limit_splits_groups():
    g = Graph()
    xs = [g.input(f"x{i}", "f32", (2, 8)) for i in range(21)]
    v = xs[0]
    for i in range(20):
        v = g.op("add", [v, xs[i + 1]], f"s{i}", "f32", (2, 8), role="out" if i == 19 else "tmp")
    # a group of m chained adds reads m+1 inputs and writes one output: m <= 14
    assert [len(x) for x in pt.partition(g)] == [14, 6]


def test_graph_output_in_the_middle_cuts_post_dominance():
    g = Graph()
    x = g.input("x", "f32", (4, 8))
    a = g.op("exp", [x], "a", "f32", (4, 8))
    b = g.op("neg", [a], "b", "f32", (4, 8), role="out")
    g.op("relu", [b], "c", "f32", (4, 8), role="out")
    assert pt.immediate_postdominators(g) == [1, None, None]
    assert as_sets(pt.partition(g)) == [[0, 1], [2]]


# ---------------------------------------------------- brute-force post-dominators
def _paths_to_exit(g, succ, i):
    out = []

    def walk(v, path):
        if pt.exits_to_end(g, v, succ):
            out.append(path + [v])
        for s in succ[v]:
            walk(s, path + [v])
    walk(i, [])
    return out


def _random_dags(seed, count, max_ops):
    rng = np.random.default_rng(seed)
    unary = ["exp", "neg", "relu", "square"]
    for _ in range(count):
        n = int(rng.integers(1, max_ops + 1))
        g = Graph()
        avail = [g.input("x0", "f32", (3, 5)), g.input("x1", "f32", (3, 5))]
        for i in range(n):
            k = int(rng.integers(1, 4))
            ins = [avail[int(j)] for j in rng.integers(0, len(avail), size=k)]
            op = {1: unary[int(rng.integers(0, 4))], 2: "add", 3: "add3"}[k]
            avail.append(g.op(op, ins, f"t{i}", "f32", (3, 5)))
        readers = {t for o in g.ops for t in o.inputs}
        # every unread result is an output; some read ones too
        for o in g.ops:
            t = o.output
            if t not in readers or rng.random() < 0.15:
                g.tensors[t] = TensorDesc(g.tensors[t].name, "f32", (3, 5), "out")
        yield g


def test_postdominators_match_path_enumeration():
    for g in _random_dags(11, 600, 7):
        succ = pt.successors(g)
        sets = pt.postdominator_sets(g)
        for i in range(len(g.ops)):
            paths = _paths_to_exit(g, succ, i)
            on_all = set.intersection(*[set(p) for p in paths]) - {i}
            assert sets[i] - {i, -1} == on_all
            ipd = pt.immediate_postdominators(g)[i]
            if on_all:
                # the nearest one comes first on every path
                firsts = {next(v for v in p[1:] if v in on_all) for p in paths}
                assert firsts == {ipd}
            else:
                assert ipd is None


def test_groups_are_convex_and_rule_abiding_on_random_dags():
    for g in _random_dags(12, 400, 7):
        groups = pt.partition(g)
        succ = pt.successors(g)
        owner = {i: gi for gi, grp in enumerate(groups) for i in grp}
        for grp in groups:
            s = set(grp)
            # convex: nothing outside the group lies on a path between members
            for a, b in itertools.permutations(grp, 2):
                reach_a = pt._reach(succ, a)
                for v in reach_a:
                    if v not in s and b in pt._reach(succ, v):
                        raise AssertionError((grp, a, b, v))
            assert len(grp) <= pt.MAX_FUSED_OPS
        # groups are listed in an order that respects dependencies
        for gi, grp in enumerate(groups):
            for i in grp:
                for s2 in succ[i]:
                    assert owner[s2] >= gi


# ---------------------------------------------------------------- row-resident extension
def _rr_graphs():
    """Graphs for the row-resident merge: name -> (graph, groups without
    the extension, groups with it)."""
    out = {}
    g = configs.layernorm_graph(16, 64)
    out["layernorm"] = (g, [[0], [1, 2, 3], [4, 5, 6, 7, 8, 9, 10]], [list(range(11))])
    g = Graph()
    x = g.input("x", "f32", (8, 40))
    s = g.op("row_sum", [x], "s", "f32", (8, 1))
    g.op("mul", [x, s], "y", "f32", (8, 40), role="out")
    out["scale_by_sum"] = (g, [[0], [1]], [[0, 1]])
    g = Graph()
    x = g.input("x", "f32", (8, 40))
    e = g.op("exp", [x], "e", "f32", (8, 40))
    s = g.op("row_sum", [e], "s", "f32", (8, 1))
    g.op("div", [e, s], "y", "f32", (8, 40), role="out")
    out["softmax_like"] = (g, [[0], [1], [2]], [[0], [1, 2]])
    out["softmax"] = (configs.softmax_graph(16, 64), [[0], [1, 2, 3], [4, 5, 6, 7]], [list(range(8))])
    g = Graph()
    x = g.input("x", "f32", (8, 40))
    g.op("row_mean", [x], "m", "f32", (8, 1), role="out")
    out["reduce_only"] = (g, [[0]], [[0]])
    g = Graph()
    x = g.input("x", "f32", (8, 40))
    s = g.op("row_sum", [x], "s", "f32", (8, 1))
    u = g.op("copy", [s], "u", "f32", (8, 1), opaque=True)
    t = g.op("mul", [x, s], "t", "f32", (8, 40))
    g.op("add", [t, u], "y", "f32", (8, 40), role="out")
    out["opaque_on_path"] = (g, [[0], [1], [2, 3]], [[0], [1], [2, 3]])
    g = Graph()
    v = g.input("x", "f32", (8, 40))
    for k in range(6):
        m = g.op("row_mean", [v], f"m{k}", "f32", (8, 1))
        v = g.op("sub", [v, m], f"c{k}", "f32", (8, 40), role="out" if k == 5 else "tmp")
    out["six_reductions"] = (g, None, None)
    return out


def test_row_resident_merges():
    for name, (g, plain, merged) in _rr_graphs().items():
        if plain is None:
            continue
        assert pt.partition(g) == plain, name
        assert pt.partition(g, row_resident=True) == merged, name


def test_row_resident_merge_keeps_the_group_graph_acyclic():
    """The row-resident merge's own rules (beyond TVM's limits) are
    convexity and nothing else: a reduction read through an opaque op and
    directly stays apart where merging would put the opaque op on a path
    out of and back into the group."""
    g, plain, merged = _rr_graphs()["opaque_on_path"]
    assert pt.partition(g, row_resident=True) == merged
    for grp in pt.partition(g, row_resident=True):
        succ = pt.successors(g)
        assert pt._convex(succ, set(grp))


# ---------------------------------------------------------------- duplicate fusion
def _canon(g):
    """Each op's value as an expression tree over the graph's named inputs,
    so graphs that compute the same things in another op order compare
    equal."""
    prod = {o.output: i for i, o in enumerate(g.ops)}
    memo = {}

    def of(t):
        if t not in prod:
            return ("in", g.tensors[t].name)
        if t not in memo:
            o = g.ops[prod[t]]
            memo[t] = (o.op, o.imm, g.tensors[t].dtype, tuple(of(x) for x in o.inputs))
        return memo[t]
    return [of(o.output) for o in g.ops], of


def test_plan_cost_counts_bytes_by_hand():
    # c2: one group reading X, bias, R and writing y (bf16 [4,16], bias [16])
    g = configs.c2_graph(4, 16)
    assert pt.plan_cost(g, pt.partition(g)) == (2 * (3 * 64 + 16), 1)
    # unfused: bias_add writes t (read by relu), relu writes u (read by add)
    assert pt.plan_cost(g, pt.partition(g, fuse=False)) == (2 * (64 + 16 + 64) + 2 * (64 + 64)
                                                            + 2 * (64 + 64 + 64), 3)


def test_duplicate_layernorm_is_the_hand_duplicated_layernorm():
    """x - mean written once is recomputed in both groups that read it: the
    result computes exactly what the descriptor with x - mean written twice
    computes, in the same three groups, at the same cost."""
    for rr in (False, True):
        shared = configs.layernorm_shared_graph(16, 64)
        hand = configs.layernorm_graph(16, 64)
        g2, origin = pt.duplicate(shared, row_resident=rr)
        assert len(pt.partition(shared, row_resident=rr)) == (4 if not rr else 2)
        ops2, of2 = _canon(g2)
        opsh, ofh = _canon(hand)
        assert sorted(map(repr, ops2)) == sorted(map(repr, opsh))
        groups2 = {frozenset(repr(ops2[i]) for i in grp) for grp in pt.partition(g2, row_resident=rr)}
        groupsh = {frozenset(repr(opsh[i]) for i in grp) for grp in pt.partition(hand, row_resident=rr)}
        assert groups2 == groupsh
        assert pt.plan_cost(g2, pt.partition(g2, row_resident=rr)) == \
            pt.plan_cost(hand, pt.partition(hand, row_resident=rr))
        # the copy of x - mean computes op 1 of the shared graph; the shared op is gone
        assert origin.count(1) == 2 and len(g2.ops) == len(shared.ops) + 1
        for i, o in enumerate(g2.ops):
            assert (o.op, o.imm) == (shared.ops[origin[i]].op, shared.ops[origin[i]].imm)


def test_duplicate_is_not_kept_when_it_moves_more_bytes():
    """p = a + b (f32 inputs, bf16 result) read by three row sums in three
    groups: recomputing p in each reads 8 bytes per element three times
    instead of storing 2 and reading them back three times."""
    g = Graph()
    a = g.input("a", "f32", (8, 32))
    b = g.input("b", "f32", (8, 32))
    p = g.op("add", [a, b], "p", "bf16", (8, 32))
    for k in range(3):
        g.op("row_sum", [p], f"s{k}", "f32", (8, 1), role="out")
    g2, origin = pt.duplicate(g)
    assert g2 is g and origin == [0, 1, 2, 3]
    # with a bf16 input and an f32 result the same rewrite pays off
    h = Graph()
    a = h.input("a", "bf16", (8, 32))
    p = h.op("exp", [a], "p", "f32", (8, 32))
    for k in range(3):
        h.op("row_sum", [p], f"s{k}", "f32", (8, 1), role="out")
    h2, origin = pt.duplicate(h)
    assert origin == [0, 1, 0, 2, 0, 3] and len(pt.partition(h2)) == 3
    assert pt.plan_cost(h2, pt.partition(h2)) == (3 * (2 * 256 + 4 * 8), 3)


def test_duplicate_leaves_readers_in_the_same_group_alone():
    g = configs.c3_graph(8, 64, head_op=True)  # the head's three readers share its group
    g2, origin = pt.duplicate(g)
    assert g2 is g and origin == list(range(len(g.ops)))


def _f32_reduce_dags(seed, count):
    """Small all-f32 DAGs with row sums, row and column operands and opaque
    ops: values crossing groups are stored without rounding, so a
    duplicated program computes the same bits."""
    rng = np.random.default_rng(seed)
    R, C = 3, 5
    for _ in range(count):
        g = Graph()
        full = [g.input("x0", "f32", (R, C)), g.input("x1", "f32", (R, C))]
        rowv = [g.input("r0", "f32", (R, 1))]
        col = g.input("c0", "f32", (C,))
        for i in range(int(rng.integers(2, 9))):
            kind = int(rng.integers(0, 6))
            pick = lambda xs: xs[int(rng.integers(len(xs)))]  # noqa: E731
            if kind == 0:
                full.append(g.op(["exp", "relu", "neg", "square"][int(rng.integers(4))], [pick(full)],
                                 f"t{i}", "f32", (R, C), opaque=bool(rng.random() < 0.1)))
            elif kind == 1:
                full.append(g.op(["add", "mul", "sub"][int(rng.integers(3))], [pick(full), pick(full)],
                                 f"t{i}", "f32", (R, C)))
            elif kind == 2:
                full.append(g.op("add", [pick(full), col], f"t{i}", "f32", (R, C)))
            elif kind == 3:
                full.append(g.op("mul", [pick(full), pick(rowv)], f"t{i}", "f32", (R, C)))
            elif kind == 4:
                red = "row_max" if i % 3 == 1 else "row_sum"   # no draw: the DAGs stay as they were
                rowv.append(g.op(red, [pick(full)], f"t{i}", "f32", (R, 1)))
            else:
                rowv.append(g.op("add_imm", [pick(rowv)], f"t{i}", "f32", (R, 1), imm=0.5))
        readers = {t for o in g.ops for t in o.inputs}
        for o in g.ops:
            t = o.output
            if t not in readers or rng.random() < 0.1:
                d = g.tensors[t]
                g.tensors[t] = TensorDesc(d.name, d.dtype, d.shape, "out")
        yield g


def test_duplicate_preserves_values_and_never_raises_the_cost():
    from oracle import evaluate as oev
    changed = 0
    for k, g in enumerate(_f32_reduce_dags(23, 400)):
        for rr in (False, True):
            g2, origin = pt.duplicate(g, row_resident=rr)
            p1, p2 = pt.partition(g, row_resident=rr), pt.partition(g2, row_resident=rr)
            assert pt.plan_cost(g2, p2) <= pt.plan_cost(g, p1)
            if g2 is g:
                continue
            changed += 1
            assert pt.plan_cost(g2, p2) < pt.plan_cost(g, p1)
            assert g2.tensors[:len(g.tensors)] == g.tensors
            for i, o in enumerate(g2.ops):
                src = g.ops[origin[i]]
                assert (o.op, o.imm, o.opaque) == (src.op, src.imm, src.opaque)
                assert g2.tensors[o.output].shape == g.tensors[src.output].shape
            # every copy shares a group with its single reader
            gof = {i: j for j, grp in enumerate(p2) for i in grp}
            for i, o in enumerate(g2.ops):
                if o.output >= len(g.tensors):
                    rd = [j for j, q in enumerate(g2.ops) if o.output in q.inputs]
                    assert len(rd) == 1 and rd[0] > i and gof[i] == gof[rd[0]]
            ins = {}
            for j, t in enumerate(g.inputs()):
                ins[t] = configs.tensor_values("f32", g.tensors[t].shape, "uniform", 900 + k, j, -1.5, 1.5)
            _, want = oev.run(g, ins, stored=pt.stored_tensors(g, p1), groups=p1)
            _, got = oev.run(g2, ins, stored=pt.stored_tensors(g2, p2), groups=p2)
            for t in g.outputs():
                assert np.array_equal(got[t].view(np.uint32), want[t].view(np.uint32))
    assert changed >= 30


def test_values_read_inside_their_group_are_not_rounded():
    """Inside a group every intermediate is fp32; rounding to the tensor's
    dtype happens at the store.  a = x / 3 is a bf16 graph output that b
    also reads: in one group b sees the fp32 quotient, across groups the
    stored bf16 value."""
    from oracle import evaluate as oev
    from oracle import numerics
    g = Graph()
    x = g.input("x", "f32", (1, 4))
    a = g.op("mul_imm", [x], "a", "bf16", (1, 4), role="out", imm=1.0 / 3.0)
    b = g.op("mul_imm", [a], "b", "f32", (1, 4), role="out", imm=3.0)
    xs = np.array([[1.0, 2.0, 5.0, 7.0]], dtype=np.float32)
    q = (xs * np.float32(1.0 / 3.0)).astype(np.float32)
    one = oev.evaluate(g, {x: xs}, groups=[[0, 1]])
    two = oev.evaluate(g, {x: xs}, groups=[[0], [1]])
    assert np.array_equal(one[b], (q * np.float32(3.0)).astype(np.float32))
    qb = numerics.bf16_to_f32(numerics.encode(q, "bf16"))
    assert np.array_equal(two[b], (qb * np.float32(3.0)).astype(np.float32))
    assert not np.array_equal(one[b], two[b])
    # the stored output is the rounded quotient either way
    assert np.array_equal(one[a], qb.reshape(1, 4)) and np.array_equal(two[a], qb.reshape(1, 4))


# ---------------------------------------------------------------- injective data movement
def test_transpose_reshape_concat_values():
    """The oracle's transpose, reshape and concat against their
    definitions, element by element."""
    from oracle import evaluate as oev
    g = Graph()
    x = g.input("x", "f32", (3, 5))
    y = g.input("y", "bf16", (3, 2))
    t = g.op("transpose", [x], "t", "f32", (5, 3), role="out")
    r = g.op("reshape", [x], "r", "f32", (5, 3), role="out")
    v = g.op("reshape", [x], "v", "f32", (15,), role="out")
    c = g.op("concat", [x, g.input("z", "f32", (3, 2))], "c", "f32", (3, 7), role="out")
    xs = np.arange(15, dtype=np.float32).reshape(3, 5)
    zs = np.array([[100, 101], [102, 103], [104, 105]], dtype=np.float32)
    out = oev.outputs(g, oev.evaluate(g, {x: xs, y: np.zeros((3, 2), np.uint16), 5: zs}))
    for i in range(3):
        for j in range(5):
            assert out[t][j, i] == xs[i, j]                  # transpose
            assert out[r].ravel()[i * 5 + j] == xs[i, j]     # row-major order kept
            assert out[v][i * 5 + j] == xs[i, j]
            assert out[c][i, j] == xs[i, j]
        assert out[c][i, 5] == zs[i, 0] and out[c][i, 6] == zs[i, 1]
    assert [pt.pattern(g, i) for i in range(4)] == [pt.K_INJECTIVE] * 4


def test_injective_ops_fuse_by_the_phase_rules():
    # transpose -> exp: an injective source fuses in phase 1 into an
    # elementwise post-dominator
    g = Graph()
    x = g.input("x", "f32", (3, 5))
    t = g.op("transpose", [x], "t", "f32", (5, 3))
    g.op("exp", [t], "y", "f32", (5, 3), role="out")
    assert as_sets(pt.partition(g)) == [[0, 1]]
    # ... but not into a reduction (kInjective needs an injective-or-simpler sink)
    g = Graph()
    x = g.input("x", "f32", (3, 5))
    t = g.op("transpose", [x], "t", "f32", (5, 3))
    g.op("row_sum", [t], "s", "f32", (5, 1), role="out")
    assert as_sets(pt.partition(g)) == [[0], [1]]
    # exp -> transpose: the elementwise producer fuses into its injective
    # post-dominator (phase 0's rule); whether one launch can run the
    # result is the executor's matter, not the pages'
    g = Graph()
    x = g.input("x", "f32", (3, 5))
    e = g.op("exp", [x], "e", "f32", (3, 5))
    g.op("transpose", [e], "y", "f32", (5, 3), role="out")
    assert as_sets(pt.partition(g)) == [[0, 1]]
    # concat of two inputs feeding elementwise work: one group
    g = Graph()
    a = g.input("a", "f32", (4, 3))
    b = g.input("b", "f32", (4, 5))
    c = g.op("concat", [a, b], "c", "f32", (4, 8))
    g.op("relu", [c], "y", "f32", (4, 8), role="out")
    assert as_sets(pt.partition(g)) == [[0, 1]]
    # a transposed input also read directly: one group by the phases
    g = Graph()
    x = g.input("x", "f32", (4, 4))
    t = g.op("transpose", [x], "t", "f32", (4, 4))
    g.op("add", [t, x], "y", "f32", (4, 4), role="out")
    assert as_sets(pt.partition(g)) == [[0, 1]]


# ---------------------------------------------------------------- tuples (kTuple)
def _tuple_graph(field="transpose", concat_opaque=False, tail="mul_imm"):
    """y = f(concat((a, b))) with a, b fields made from inputs X [5,3] and
    Y [2,3] by `field` (transpose, or exp of [3,5] / [3,2] inputs)."""
    g = Graph()
    if field == "transpose":
        a = g.op("transpose", [g.input("X", "f32", (5, 3))], "a", "f32", (3, 5))
        b = g.op("transpose", [g.input("Y", "f32", (2, 3))], "b", "f32", (3, 2))
    else:
        a = g.op("exp", [g.input("X", "f32", (3, 5))], "a", "f32", (3, 5))
        b = g.op("transpose", [g.input("Y", "f32", (2, 3))], "b", "f32", (3, 2))
    t = g.op("tuple", [a, b], "t", "f32", (3, 7))
    c = g.op("concat", [t], "c", "f32", (3, 7), opaque=concat_opaque)
    if tail == "mul_imm":
        g.op("mul_imm", [c], "y", "f32", (3, 7), role="out", imm=0.5)
    else:   # a reshaped input added after the concat, listed after it
        r = g.op("reshape", [g.input("V", "f32", (7, 3))], "r", "f32", (3, 7))
        g.op("add", [c, r], "y", "f32", (3, 7), role="out")
    return g


def test_tuple_values_and_pattern():
    """A tuple's value is its fields side by side and the concat of it is
    that value; the table makes a tuple kTuple (7)."""
    from oracle import evaluate as oev
    g = _tuple_graph()
    xs = np.arange(15, dtype=np.float32).reshape(5, 3)
    ys = 100 + np.arange(6, dtype=np.float32).reshape(2, 3)
    out = oev.outputs(g, oev.evaluate(g, {0: xs, 2: ys}))[g.outputs()[0]]
    for i in range(3):
        assert list(out[i]) == [0.5 * v for v in list(xs[:, i]) + list(ys[:, i])]
    assert [pt.pattern(g, i) for i in range(5)] == [pt.K_INJECTIVE, pt.K_INJECTIVE, pt.K_TUPLE,
                                                    pt.K_INJECTIVE, pt.K_ELEMWISE]


def test_tuple_fuses_into_its_concat_and_its_fields_follow_in_phase_two():
    # the tuple fuses into the injective concat after it (phase 1), the
    # concat into the scaling; then the transposes, whose post-dominator
    # is the tuple, join the tuple's group in phase 2
    assert as_sets(pt.partition(_tuple_graph())) == [[0, 1, 2, 3, 4]]
    # an opaque concat keeps the tuple out of any later group, so phase 2
    # has no absorbed tuple to fuse the fields into
    assert as_sets(pt.partition(_tuple_graph(concat_opaque=True))) == [[0], [1], [2], [3], [4]]
    # phase 2 takes any field no more complex than injective: by the rules
    # the exp joins too ...
    g = _tuple_graph(field="exp")
    assert as_sets(pt.partition(g)) == [[0, 1, 2, 3, 4]]
    # ... while the executor reads a join's fields from memory, so with its
    # capacity the exp stays a group of its own
    from tests import capacity as cap
    assert as_sets(cap.partition(g)) == [[0], [1, 2, 3, 4]]


def test_a_group_holding_an_absorbed_tuple_counts_as_injective():
    """The reshape after the concat is visited in phase 1 after the tuple
    fused onward: its post-dominator's group then holds the tuple as an
    injective member, so the reshape (injective) fuses.  Were the tuple's
    kTuple kept in the group's combined pattern, the reshape would stay
    alone."""
    g = _tuple_graph(tail="reshape")
    assert as_sets(pt.partition(g)) == [[0, 1, 2, 3, 4, 5]]
