"""The executor's capacity model (tests/capacity.py), pinned against the
library's own account of the groups it runs, and the rules that are the
executor's, not the pages': checked here with the model composed into the
oracle's grouping, where the oracle's own rules would fuse further."""
import numpy as np
import pytest

import gradient_tensor_fusion_amd as gtf
from gradient_tensor_fusion_amd import _capi as C
from oracle import partition as pt
from oracle import search as sr
from tests import capacity as cap
from tests.test_capi_host import _broadcast_dags
from tests.test_oracle_partition import _f32_reduce_dags
from workloads import configs
from workloads.graph import Graph


def as_sets(groups):
    return sorted(sorted(x) for x in groups)


def _random_groupings(seed):
    """(graph, labels) pairs: random labelings and merges of fusion-pass
    groups of random broadcast and reduction DAGs, and the LayerNorms."""
    rng = np.random.default_rng(seed)
    graphs = list(_f32_reduce_dags(seed, 120)) + list(_broadcast_dags(seed + 1, 120))
    graphs += [configs.layernorm_graph(16, 64), configs.layernorm_shared_graph(16, 64),
               configs.softmax_graph(16, 64)]
    for g in graphs:
        n = len(g.ops)
        labs = [list(rng.integers(0, max(1, n // 2 + 1), size=n)) for _ in range(4)]
        groups = pt.partition(g, row_resident=True)
        lab = [0] * n
        for k, grp in enumerate(groups):
            for i in grp:
                lab[i] = k
        labs.append(lab)
        yield from ((g, [int(x) for x in lb]) for lb in labs)


def test_layout_matches_the_library_geometry():
    """For every group of every random grouping the library accepts, the
    model's layout equals what fuse_plan_group_geometry and
    fuse_plan_group_tensors report: the element stages, the tensors read or
    written in memory, and the LDS bytes (4 bytes per column of each
    column slot, per row of each row slot, and a 64-byte reduce buffer)."""
    n_groups = n_multi = 0
    for g, lab in _random_groupings(501):
        try:
            plan = gtf.FusePlan.grouped(g, lab)
        except gtf.GtfError as e:
            assert e.status == C.GTF_E_INVALID
            continue
        for k in range(plan.num_groups):
            ops = plan.group_ops(k)
            lay = cap.layout(g, set(ops))
            assert lay is not None, ops
            geo = plan.geometry(k)
            assert geo["stages"] == lay["stages"], (ops, geo, lay)
            assert len(plan.group_tensors(k)) == lay["slots"], (ops, lay)
            want = 4 * (lay["col_slots"] * geo["panel_width"] + lay["row_slots"] * geo["rows_per_item"] + 16)
            assert geo["lds_bytes"] == want, (ops, geo, lay)
            n_groups += 1
            n_multi += lay["stages"] > 1
    assert n_groups >= 500 and n_multi >= 50


def test_group_ok_is_what_the_library_accepts():
    """Every group of a grouping the library accepts passes group_ok, and a
    grouping whose groups all pass it (and which is a valid plan by the
    page's rules) is accepted."""
    for g, lab in _random_groupings(502):
        ok_model = sr.plan_ok(g, lab, cap.group_ok)
        try:
            gtf.FusePlan.grouped(g, lab)
            ok_lib = True
        except gtf.GtfError:
            ok_lib = False
        assert ok_lib == ok_model, lab


def test_moves_run_only_as_loads():
    """TVM's phases fuse an elementwise producer into a transpose, and a
    transpose into a reader of its input; the executor reads a transpose's
    input from memory, so with the model composed in these stay apart."""
    g = Graph()
    x = g.input("x", "f32", (3, 5))
    e = g.op("exp", [x], "e", "f32", (3, 5))
    g.op("transpose", [e], "y", "f32", (5, 3), role="out")
    assert as_sets(pt.partition(g)) == [[0, 1]]          # the pages' rules
    assert as_sets(cap.partition(g)) == [[0], [1]]       # what one launch runs
    assert as_sets(gtf.FusePlan(g).groups()) == [[0], [1]]
    g = Graph()
    x = g.input("x", "f32", (4, 4))
    t = g.op("transpose", [x], "t", "f32", (4, 4))
    g.op("add", [t, x], "y", "f32", (4, 4), role="out")
    assert as_sets(pt.partition(g)) == [[0, 1]]
    assert as_sets(cap.partition(g)) == [[0], [1]]
    assert as_sets(gtf.FusePlan(g).groups()) == [[0], [1]]


def test_stage_limit_of_the_row_resident_merge():
    """m_0 = mean(x), m_{k+1} = mean((x - m_k)^2): TVM's phases group each
    (x - m_k, its square, m_{k+1}), and the oracle's row-resident merge
    alone chains them all into one group.  The executor holds at most four
    stages (m_0 and m_1 pair into one), so with the model composed in the
    chain splits, every group within the limit, as the library's plan does."""
    g = Graph()
    x = g.input("x", "f32", (8, 40))
    m = g.op("row_mean", [x], "m0", "f32", (8, 1))
    for k in range(6):
        d = g.op("sub", [x, m], f"d{k}", "f32", (8, 40))
        q = g.op("square", [d], f"q{k}", "f32", (8, 40))
        m = g.op("row_mean", [q], f"m{k + 1}", "f32", (8, 1), role="out" if k == 5 else "tmp")
    assert len(pt.partition(g)) == 7
    assert len(pt.partition(g, row_resident=True)) == 1
    groups = cap.partition(g, row_resident=True)
    assert 1 < len(groups) < 7
    for grp in groups:
        assert cap.layout(g, set(grp))["stages"] <= cap.MAX_STAGES
    assert max(cap.layout(g, set(grp))["stages"] for grp in groups) == cap.MAX_STAGES
    plan = gtf.FusePlan(g, row_resident=True)
    assert as_sets(plan.groups()) == as_sets(groups)
    assert max(plan.geometry(k)["stages"] for k in range(plan.num_groups)) == cap.MAX_STAGES


def test_capacity_rules_on_hand_groupings():
    """A [1,C] op after a reduction of its group, and two reductions ending
    one stage, are valid plans by the pages' rules and beyond the executor."""
    g = Graph()
    x = g.input("x", "f32", (4, 8))
    c = g.input("c", "f32", (8,))
    s = g.op("row_sum", [x], "s", "f32", (4, 1))
    y = g.op("mul", [x, s], "y", "f32", (4, 8))
    g.op("add", [y, c], "z", "f32", (4, 8), role="out")
    assert sr.plan_ok(g, [0, 0, 0]) and sr.plan_ok(g, [0, 0, 0], cap.group_ok)
    g2 = Graph()
    x = g2.input("x", "f32", (4, 8))
    s = g2.op("row_sum", [x], "s", "f32", (4, 1))
    m = g2.op("row_mean", [x], "m", "f32", (4, 1))
    g2.op("add", [s, m], "t", "f32", (4, 1), role="out")
    assert sr.plan_ok(g2, [0, 0, 1])
    assert not sr.plan_ok(g2, [0, 0, 1], cap.group_ok)
    with pytest.raises(gtf.GtfError):
        gtf.FusePlan.grouped(g2, [0, 0, 1])
    g3 = Graph()
    x = g3.input("x", "f32", (4, 8))
    s = g3.op("row_sum", [x], "s", "f32", (4, 1))
    cc = g3.op("exp", [g3.input("c", "f32", (8,))], "cc", "f32", (8,))
    g3.op("add", [s, cc], "t", "f32", (4, 8), role="out")
    assert sr.plan_ok(g3, [0, 0, 0])
    assert cap.layout(g3, {0, 1, 2}) is not None


def test_opaque_ops_are_never_fused():
    """DisCo's plans never fuse a parameter or control-flow op: the oracle's
    validity rule and the library both refuse a group that holds an opaque
    op with another."""
    g = Graph()
    x = g.input("x", "f32", (4, 8))
    a = g.op("exp", [x], "a", "f32", (4, 8))
    b = g.op("copy", [a], "b", "f32", (4, 8), opaque=True)
    g.op("relu", [b], "y", "f32", (4, 8), role="out")
    assert sr.plan_ok(g, [0, 1, 2]) and not sr.plan_ok(g, [0, 0, 1]) and not sr.plan_ok(g, [0, 1, 1])
    for lab in ([0, 0, 1], [0, 1, 1]):
        with pytest.raises(gtf.GtfError, match="opaque"):
            gtf.FusePlan.grouped(g, lab)
    gtf.FusePlan.grouped(g, [0, 1, 2])
