"""The group compiler's programs replayed on the host (tests/program_replay.py)
against the oracle's evaluation of the same plan, within the per-element
bound the GPU parity tests use (bit-exact wherever only IEEE operations
lead to a value).  A wrong register, spill slot, LDS slot, form or stage in
a compiled program changes a result here, on the CPU, before any launch:
the workloads at small shapes, every DAG of two ops, random DAGs over
every opcode, broadcast and row-resident groups, duplicated producers,
explicit groupings, the addressed loads (transpose, concat, reshape) and
tuples with their moves folded into the concat load."""
import numpy as np
import pytest

import gradient_tensor_fusion_amd as gtf
from tests import capacity as cap
from tests import dag_gen
from tests.error_bound import assert_within, run_with_bounds
from tests.program_replay import NAME, replay_plan
from workloads import configs
from workloads.graph import Graph

SHAPES = [(1, 1), (3, 5), (2, 67), (5, 130)]


def _inputs_for(g, seed):
    """Seeded inputs: values uniform on [-1.5, 1.5) (bf16 rounded where the
    tensor is bf16), masks keep 0.9."""
    ins = {}
    for k, t in enumerate(g.inputs()):
        d = g.tensors[t]
        if d.dtype == "u8":
            u = configs.tensor_values("f32", d.shape, "uniform", seed, k, 0.0, 1.0)
            ins[t] = (u >= 0.1).astype(np.uint8)
            continue
        x = configs.tensor_values("f32", d.shape, "uniform", seed, k, -1.5, 1.5)
        ins[t] = configs.to_bf16_bits(x.astype(np.float64)) if d.dtype == "bf16" else x
    return ins


def _reshape(g, R, C):
    """The same graph with [3,5]-family shapes replaced by [R, C]."""
    m = {(3, 5): (R, C), (3, 1): (R, 1), (5,): (C,)}
    out = Graph()
    for d in g.tensors:
        out.tensors.append(type(d)(d.name, d.dtype, m.get(d.shape, d.shape), d.role))
    out.ops = list(g.ops)
    return out


def check(g, ins, plan=None, **kw):
    """Replay the plan; its outputs within the bound of the oracle's
    evaluation of the plan's own program under the plan's grouping."""
    plan = plan or gtf.FusePlan(g, **kw)
    got = replay_plan(g, plan, ins)
    vals, bound = run_with_bounds(plan.program(), ins, plan.groups())
    for t in g.outputs():
        assert_within(got[t], vals[t], bound[t], g.tensors[t].dtype, g.tensors[t].name)
    return plan


def _forms_used(plan):
    return {NAME[f] for g in range(plan.num_groups) for f, _, _ in plan.code(g)["instr"]}


def test_replay_reads_the_executors_form_table():
    # the enumeration parsed from the executor's header, in its order
    assert NAME[0] == "LD_F32_A" and "RED_SE" in NAME.values()
    assert sorted(NAME) == list(range(len(NAME)))


def test_program_view_matches_the_geometry():
    g = configs.layernorm_graph(37, 1024)
    for rr in (False, True):
        plan = gtf.FusePlan(g, row_resident=rr)
        for k in range(plan.num_groups):
            code, geo = plan.code(k), plan.geometry(k)
            assert len(code["instr"]) == geo["program_length"]
            assert len(code["stages"]) == geo["stages"]
            kinds = [st["reduce"] for st in code["stages"] if st["reduce"]]
            assert geo["reduce"] == (kinds[-1] if kinds else 0)


@pytest.mark.parametrize("rr", [False, True])
def test_workloads_at_small_shapes(rr):
    cases = [
        (configs.c1_graph(64, 512), configs.c1_inputs),
        (configs.c2_graph(64, 1000), configs.c2_inputs),
        (configs.c3_graph(33, 1024), configs.c3_inputs),
        (configs.c3_graph(5, 130, head_op=True), configs.c3_inputs),
        (configs.layernorm_graph(37, 1024), lambda g: configs.layernorm_inputs(g, 7)),
        (configs.softmax_graph(37, 1000), lambda g: configs.softmax_inputs(g, 8)),
        (configs.gelu_graph(9, 4096), lambda g: configs.gelu_inputs(g, 9)),
        (configs.dropout_graph(11, 1000), lambda g: configs.dropout_inputs(g, 10)),
        (configs.grad_epilogue_graph(1000), lambda g: configs.grad_epilogue_inputs(g, 0)),
    ]
    for g, mk in cases:
        check(g, mk(g), row_resident=rr)
        check(g, mk(g), fuse=False)


def test_c3_sums_each_term_of_the_diamond():
    """The diamond's sum runs as one reduction fed term by term: the
    element program folds three values and stores nothing else.  Its one
    input, read three times, is loaded into B and read there by the exp,
    the scaling and the tanh: no register move."""
    g = configs.c3_graph(33, 1024)
    plan = check(g, configs.c3_inputs(g))
    assert plan.num_groups == 1
    names = [NAME[f] for f, _, _ in plan.code(0)["instr"]]
    assert names.count("RED") == 3 and not any(n.startswith("ST_") for n in names)
    assert names == ["LD_BF16_B", "EXP_B", "RED", "MUL_IB", "RED", "TANH_B", "RED"], names


def test_random_elementwise_dags():
    from tests.test_oracle_partition import _random_dags
    for gi, g in enumerate(_random_dags(31, 40, 4)):
        for R, C in SHAPES:
            gg = _reshape(g, R, C)
            ins = _inputs_for(gg, 100 + gi)
            check(gg, ins)
            check(gg, ins, fuse=False)


@pytest.mark.parametrize("shape", [(3, 5), (2, 67)])
def test_every_dag_of_two_ops(shape):
    dags = dag_gen.exhaustive_small()
    for c0 in range(0, len(dags), 800):
        g, _ = dag_gen.combine(dags[c0:c0 + 800], shape)
        ins = _inputs_for(g, 1300 + c0)
        check(g, ins)
        check(g, ins, fuse=False)


def test_every_connected_dag_of_three_ops():
    dags = dag_gen.exhaustive_three()
    assert len(dags) == 1000
    for c0 in range(0, len(dags), 500):
        g, _ = dag_gen.combine(dags[c0:c0 + 500], (5, 130))
        ins = _inputs_for(g, 1500 + c0)
        check(g, ins)
        check(g, ins, fuse=False)


def test_random_dags_over_every_opcode():
    used = set()
    for n_ops in (3, 6, 10, 16):
        for k, g in enumerate(dag_gen.random_dags(40 + n_ops, 30, n_ops)):
            for shape in ((3, 5), (5, 130)):
                gg = _reshape(g, *shape)
                used |= _forms_used(check(gg, _inputs_for(gg, 1700 + k)))
    # every elementwise form and the spill moves of the wide and narrow
    # instances came up
    for f in ("EXP", "TANH", "SIGMOID", "RELU", "GELU", "SQUARE", "SQRT", "RECIP", "NEG", "ADD",
              "SUB", "MUL", "DIV", "MAX", "MIN", "A2S0", "S02B"):
        assert f in used, f


def _broadcast_dags(seed, count):
    from tests.test_capi_host import _broadcast_dags as bd
    return bd(seed, count)


@pytest.mark.parametrize("rr", [False, True])
def test_random_broadcast_dags(rr):
    n = 0
    for gi, g in enumerate(_broadcast_dags(7, 200)):
        for R, C in [(3, 5), (2, 67), (300, 24)]:
            gg = _reshape(g, R, C)
            check(gg, _inputs_for(gg, 200 + gi), row_resident=rr)
            n += 1
    assert n == 600


def test_random_dags_with_duplicate_fusion():
    from tests.test_oracle_partition import _f32_reduce_dags
    for gi, g in enumerate(list(_f32_reduce_dags(23, 120)) + list(_broadcast_dags(31, 120))):
        for R, C in [(3, 5), (300, 24)]:
            gg = _reshape(g, R, C)
            ins = _inputs_for(gg, 500 + gi)
            check(gg, ins, duplicate=True)
            check(gg, ins, duplicate=True, row_resident=True)


def test_random_grouped_plans():
    from oracle import search as osr
    from tests.test_oracle_partition import _f32_reduce_dags
    rng = np.random.default_rng(91)
    n = 0
    for gi, g in enumerate(list(_f32_reduce_dags(65, 80)) + list(_broadcast_dags(66, 80))):
        for R, C in [(3, 5), (300, 24)]:
            gg = _reshape(g, R, C)
            m = len(gg.ops)
            for _ in range(4):
                lab = [int(x) for x in rng.integers(0, max(1, m // 2 + 1), size=m)]
                if osr.plan_ok(gg, lab, cap.group_ok):
                    check(gg, _inputs_for(gg, 800 + gi), plan=gtf.FusePlan.grouped(gg, lab))
                    n += 1
    assert n >= 100


def test_random_gather_dags():
    from tests.test_capi_host import _gather_dags
    for gi, g in enumerate(_gather_dags(72, 80)):
        for R, C in [(3, 5), (40, 24), (7, 130)]:
            shape = {(3, 5): (R, C), (5, 3): (C, R), (3, 2): (R, 2), (3, 7): (R, C + 2),
                     (3, 1): (R, 1), (5, 1): (C, 1)}
            gg = Graph()
            for d in g.tensors:
                gg.tensors.append(type(d)(d.name, d.dtype, shape.get(d.shape, d.shape), d.role))
            gg.ops = list(g.ops)
            check(gg, _inputs_for(gg, 900 + gi))


def test_transpose_concat_and_reshape_groups():
    g = Graph()
    X = g.input("X", "bf16", (40, 24))
    b = g.input("b", "bf16", (40,))
    t = g.op("transpose", [X], "t", "bf16", (24, 40))
    u = g.op("add", [t, b], "u", "bf16", (24, 40))
    g.op("gelu", [u], "y", "bf16", (24, 40), role="out")
    assert "LDT_A" in _forms_used(check(g, _inputs_for(g, 950)))
    h = Graph()
    a = h.input("a", "f32", (37, 5))
    c = h.op("concat", [a, h.input("b", "f32", (37, 130))], "c", "f32", (37, 135))
    h.op("mul_imm", [c], "y", "f32", (37, 135), role="out", imm=0.5)
    assert "LDC_F32_A" in _forms_used(check(h, _inputs_for(h, 960)))
    k = Graph()
    x = k.input("x", "f32", (37, 135))
    r = k.op("reshape", [x], "r", "f32", (135, 37))
    k.op("add", [r, k.input("v", "f32", (135, 1))], "y", "f32", (135, 37), role="out")
    check(k, _inputs_for(k, 961))


@pytest.mark.parametrize("shape", [(3, 5, 2), (40, 24, 7), (7, 130, 1), (1, 1, 1), (96, 64, 33)])
def test_random_tuple_dags(shape):
    from tests.test_capi_host import _tuple_dags
    for gi, g in enumerate(_tuple_dags(82, 60, *shape)):
        ins = _inputs_for(g, 1900 + gi)
        check(g, ins)
        check(g, ins, fuse=False)


def test_tuple_of_transposes_is_one_concat_load():
    """concat((transpose(X), transpose(Y))) scaled: one group whose program
    reads both fields through one concat load at the transposes'
    addressing; neither transpose runs on its own."""
    g = Graph()
    X = g.input("X", "bf16", (24, 40))
    Y = g.input("Y", "bf16", (9, 40))
    a = g.op("transpose", [X], "a", "bf16", (40, 24))
    b = g.op("transpose", [Y], "b", "bf16", (40, 9))
    t = g.op("tuple", [a, b], "t", "bf16", (40, 33))
    c = g.op("concat", [t], "c", "bf16", (40, 33))
    g.op("mul_imm", [c], "y", "bf16", (40, 33), role="out", imm=0.5)
    plan = check(g, _inputs_for(g, 1950))
    assert plan.num_groups == 1
    names = [NAME[f] for f, _, _ in plan.code(0)["instr"]]
    assert names[0] == "LDC_BF16_A" and not any(n.startswith("LDG") or n == "LDT_A" for n in names), names
    code = plan.code(0)
    assert sorted(zip(code["rstride"], code["cstride"]))[:2] == [(1, 40), (1, 40)]


def test_grouped_and_searched_tuple_plans():
    """Random valid groupings of tuple graphs and byte-cost search results
    replay to the oracle's values on the same program and grouping."""
    from oracle import search as osr
    from tests.test_capi_host import _lib_bytes_cost, _tuple_dags
    rng = np.random.default_rng(93)
    n = 0
    for gi, g in enumerate(_tuple_dags(84, 40, 40, 24, 7)):
        m = len(g.ops)
        for _ in range(8):
            lab = [int(x) for x in rng.integers(0, max(1, m // 2 + 1), size=m)]
            if osr.plan_ok(g, lab, cap.group_ok):
                check(g, _inputs_for(g, 1960 + gi), plan=gtf.FusePlan.grouped(g, lab))
                n += 1
        if gi % 4 == 0:
            plan, _ = gtf.search(g, _lib_bytes_cost, seed=gi, max_stall=60)
            check(g, _inputs_for(g, 1980 + gi), plan=plan)
    assert n >= 40
