"""Host-side checks of libgtf.so through its C ABI (no GPU needed): every
declared symbol is exported, and the native planner (annotation,
post-dominator tree, grouping, materialisation, bucket plans) agrees with
the oracle's independent implementation."""
import ctypes
import os
import re

import numpy as np
import pytest

import gradient_tensor_fusion_amd as gtf
from gradient_tensor_fusion_amd import _capi as C
from tests import capacity as cap
from oracle import bucket as obucket
from oracle import partition as opart
from workloads import configs
from workloads.graph import Graph, OpDesc, TensorDesc
from tests.test_oracle_partition import _random_dags

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    with open(os.path.join(ROOT, "include", "gtf.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?(?:int|void|char)\s*\*?\s*(\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 18
    lib = ctypes.CDLL(C.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(C.EXPORTED)


def as_sets(groups):
    return sorted(sorted(g) for g in groups)


def check_against_oracle(g):
    plan = gtf.FusePlan(g)
    assert as_sets(plan.groups()) == as_sets(cap.partition(g))
    pats, ipd = plan.op_info()
    assert pats == [opart.pattern(g, i) for i in range(len(g.ops))]
    assert ipd == opart.immediate_postdominators(g)
    groups = cap.partition(g)
    stored = opart.stored_tensors(g, groups)
    want = {t for t, d in enumerate(g.tensors) if d.role != "tmp"} | stored
    assert set(plan.materialized()) == want
    # groups come in an order that respects their dependencies
    owner = {}
    for gi, grp in enumerate(plan.groups()):
        for i in grp:
            owner[g.ops[i].output] = gi
    for gi, grp in enumerate(plan.groups()):
        for i in grp:
            for t in g.ops[i].inputs:
                assert owner.get(t, -1) <= gi
    unf = gtf.FusePlan(g, fuse=False)
    assert as_sets(unf.groups()) == [[i] for i in range(len(g.ops))]


@pytest.mark.parametrize("make", [
    lambda: configs.c1_graph(4, 8), lambda: configs.c2_graph(4, 8),
    lambda: configs.c3_graph(4, 8), lambda: configs.c3_graph(4, 8, head_op=True),
    lambda: configs.layernorm_graph(4, 8), lambda: configs.gelu_graph(4, 8),
    lambda: configs.dropout_graph(4, 8), lambda: configs.softmax_graph(4, 8)])
def test_config_graphs_plan_like_the_oracle(make):
    check_against_oracle(make())


def test_tvm_example_and_limits_plan_like_the_oracle():
    from tests.test_oracle_partition import graph_from_json, GOLDEN
    import json
    with open(os.path.join(GOLDEN, "tvm_add_exp_squeeze.json")) as f:
        check_against_oracle(graph_from_json(json.load(f)))
    g = Graph()
    v = g.input("x", "f32", (2, 8))
    for i in range(300):
        v = g.op("neg", [v], f"t{i}", "f32", (2, 8), role="out" if i == 299 else "tmp")
    plan = gtf.FusePlan(g)
    assert [len(x) for x in plan.groups()] == [256, 44]
    check_against_oracle(g)
    g = Graph()
    xs = [g.input(f"x{i}", "f32", (2, 8)) for i in range(21)]
    v = xs[0]
    for i in range(20):
        v = g.op("add", [v, xs[i + 1]], f"s{i}", "f32", (2, 8), role="out" if i == 19 else "tmp")
    assert [len(x) for x in gtf.FusePlan(g).groups()] == [14, 6]


def test_random_dags_plan_like_the_oracle():
    for g in _random_dags(21, 300, 7):
        check_against_oracle(g)


def _broadcast_dags(seed, count):
    """Small DAGs mixing [R,C], [1,C] and [R,1] operands, reductions and
    opaque ops."""
    rng = np.random.default_rng(seed)
    R, Cc = 3, 5
    for _ in range(count):
        g = Graph()
        full = [g.input("x0", "f32", (R, Cc)), g.input("x1", "bf16", (R, Cc))]
        rowv = [g.input("r0", "f32", (R, 1))]
        colv = [g.input("c0", "bf16", (Cc,))]
        n = int(rng.integers(1, 8))
        for i in range(n):
            kind = rng.integers(0, 6)
            if kind == 0:
                a = full[rng.integers(len(full))]
                out = g.op(["exp", "relu", "neg", "tanh"][rng.integers(4)], [a], f"t{i}", "f32",
                           (R, Cc), opaque=bool(rng.random() < 0.1))
                full.append(out)
            elif kind == 1:
                a, b = full[rng.integers(len(full))], full[rng.integers(len(full))]
                full.append(g.op(["add", "mul", "sub"][rng.integers(3)], [a, b], f"t{i}", "f32", (R, Cc)))
            elif kind == 2:
                a, c = full[rng.integers(len(full))], colv[rng.integers(len(colv))]
                full.append(g.op("add", [a, c], f"t{i}", "bf16", (R, Cc)))
            elif kind == 3:
                a, r = full[rng.integers(len(full))], rowv[rng.integers(len(rowv))]
                full.append(g.op("mul", [a, r], f"t{i}", "f32", (R, Cc)))
            elif kind == 4:
                a = full[rng.integers(len(full))]
                red = "row_max" if i % 3 == 1 else "row_sum"   # no draw: the DAGs stay as they were
                rowv.append(g.op(red, [a], f"t{i}", "f32", (R, 1)))
            else:
                r = rowv[rng.integers(len(rowv))]
                rowv.append(g.op("add_imm", [r], f"t{i}", "f32", (R, 1), imm=0.5))
        readers = {t for o in g.ops for t in o.inputs}
        for o in g.ops:
            t = o.output
            if t not in readers or rng.random() < 0.1:
                d = g.tensors[t]
                g.tensors[t] = TensorDesc(d.name, d.dtype, d.shape, "out")
        yield g


def test_broadcast_dags_plan_like_the_oracle():
    for g in _broadcast_dags(5, 300):
        check_against_oracle(g)


# ------------------------------------------------------------------ errors
def _desc_status(graph_tensors, graph_ops, flags=0, version=C.ABI_VERSION):
    g = Graph(list(graph_tensors), list(graph_ops))
    desc, t, o = gtf._program_desc(g)
    desc.abi_version = version
    h = ctypes.c_void_p()
    st = C.lib().fuse_plan_create(ctypes.byref(desc), flags, ctypes.byref(h))
    if st == 0:
        C.lib().fuse_plan_destroy(h)
    else:
        assert h.value is None
    return st


T = TensorDesc


def test_descriptor_errors():
    x = T("x", "f32", (2, 3), "in")
    y = T("y", "f32", (2, 3), "out")
    ok = [OpDesc("exp", (0,), 1)]
    assert _desc_status([x, y], ok) == C.GTF_OK
    assert _desc_status([x, y], ok, version=99) == C.GTF_E_INVALID
    assert _desc_status([x, y], ok, flags=8) == C.GTF_E_INVALID
    # reads a tensor no earlier op wrote (not topological)
    tmp = T("t", "f32", (2, 3), "tmp")
    assert _desc_status([x, tmp, y], [OpDesc("exp", (1,), 2), OpDesc("exp", (0,), 1)]) == C.GTF_E_INVALID
    # bad ids
    assert _desc_status([x, y], [OpDesc("exp", (5,), 1)]) == C.GTF_E_INVALID
    assert _desc_status([x, y], [OpDesc("exp", (0,), 7)]) == C.GTF_E_INVALID
    # writes an input, writes twice, tmp nobody reads, output never written
    assert _desc_status([x, y], [OpDesc("exp", (1,), 0)]) == C.GTF_E_INVALID
    assert _desc_status([x, y], [OpDesc("exp", (0,), 1), OpDesc("neg", (0,), 1)]) == C.GTF_E_INVALID
    assert _desc_status([x, tmp, y], [OpDesc("exp", (0,), 1), OpDesc("neg", (0,), 2)]) == C.GTF_E_INVALID
    assert _desc_status([x, y], []) == C.GTF_E_INVALID
    # unsupported: u8 output
    assert _desc_status([x, T("u", "u8", (2, 3), "out")], [OpDesc("exp", (0,), 1)]) == C.GTF_E_UNSUPPORTED
    # shapes
    assert _desc_status([x, T("z", "f32", (3, 2), "in"), y], [OpDesc("add", (0, 1), 2)]) == C.GTF_E_SHAPE
    assert _desc_status([x, T("z", "f32", (2, 4), "out")], [OpDesc("exp", (0,), 1)]) == C.GTF_E_SHAPE
    assert _desc_status([x, T("s", "f32", (2,), "out")], [OpDesc("row_sum", (0,), 1)]) == C.GTF_E_SHAPE
    assert _desc_status([x, T("s", "f32", (2, 1), "out")], [OpDesc("row_sum", (0,), 1)]) == C.GTF_OK
    assert _desc_status([x, T("s", "f32", (2,), "out")], [OpDesc("row_max", (0,), 1)]) == C.GTF_E_SHAPE
    assert _desc_status([x, T("s", "f32", (2, 1), "out")], [OpDesc("row_max", (0,), 1)]) == C.GTF_OK


def test_raw_abi_errors():
    L = C.lib()
    assert L.fuse_plan_create(None, 0, ctypes.byref(ctypes.c_void_p())) == C.GTF_E_INVALID
    assert L.fuse_plan_create(None, 0, None) == C.GTF_E_INVALID
    assert b"NULL" in L.gtf_last_error()
    n = ctypes.c_int32()
    assert L.fuse_plan_num_groups(None, ctypes.byref(n)) == C.GTF_E_INVALID
    bad_op = C.ProgramDesc()
    tens = (C.TensorDesc * 2)()
    for t in tens:
        t.dtype, t.rank, t.role = 0, 2, 0
        t.shape[0], t.shape[1] = 2, 3
    tens[1].role = 1
    ops = (C.OpDesc * 1)()
    ops[0].opcode, ops[0].n_in, ops[0].out = 999, 1, 1
    desc = C.ProgramDesc(C.ABI_VERSION, 2, tens, 1, ops)
    assert L.fuse_plan_create(ctypes.byref(desc), 0, ctypes.byref(ctypes.c_void_p())) == C.GTF_E_UNSUPPORTED
    ops[0].opcode, ops[0].n_in = 1, 2
    assert L.fuse_plan_create(ctypes.byref(desc), 0, ctypes.byref(ctypes.c_void_p())) == C.GTF_E_INVALID
    tens[0].dtype = 7
    ops[0].n_in = 1
    assert L.fuse_plan_create(ctypes.byref(desc), 0, ctypes.byref(ctypes.c_void_p())) == C.GTF_E_UNSUPPORTED
    tens[0].dtype, tens[0].rank = 0, 3
    assert L.fuse_plan_create(ctypes.byref(desc), 0, ctypes.byref(ctypes.c_void_p())) == C.GTF_E_UNSUPPORTED
    tens[0].rank, tens[0].reserved = 2, 1
    assert L.fuse_plan_create(ctypes.byref(desc), 0, ctypes.byref(ctypes.c_void_p())) == C.GTF_E_INVALID
    # bucket plan errors
    arr = (ctypes.c_int64 * 2)(3, -1)
    h = ctypes.c_void_p()
    assert L.bucket_plan_create(arr, 2, 0, 64, 0, ctypes.byref(h)) == C.GTF_E_INVALID
    arr[1] = 4
    assert L.bucket_plan_create(arr, 2, 2, 64, 0, ctypes.byref(h)) == C.GTF_E_UNSUPPORTED
    assert L.bucket_plan_create(arr, 2, 0, 0, 0, ctypes.byref(h)) == C.GTF_E_INVALID
    assert L.bucket_plan_create(arr, 2, 0, 64, 1, ctypes.byref(h)) == C.GTF_E_INVALID
    assert L.bucket_plan_create(arr, 2, 0, 64, 0, ctypes.byref(h)) == C.GTF_OK
    # running before bind is a state error (checked before any device call)
    ptrs = (ctypes.c_void_p * 2)(1, 2)
    assert L.bucket_pack(h, ptrs, ptrs, 1.0, None) == C.GTF_E_STATE
    L.bucket_plan_destroy(h)


def test_bucket_plans_match_the_oracle():
    cases = [(configs.c4_numel(), 4, configs.BUCKET_CAP_BYTES),
             (configs.c5_numel(), 4, configs.BUCKET_CAP_BYTES),
             (configs.c5_numel(), 2, configs.BUCKET_CAP_BYTES)]
    rng = np.random.default_rng(3)
    for _ in range(200):
        numel = [int(v) for v in rng.integers(0, 60, size=int(rng.integers(0, 30)))]
        cases.append((numel, 4, int(rng.integers(1, 100)) * 4))
    for numel, eb, cap in cases:
        bp = gtf.BucketPlan(numel, "f32" if eb == 4 else "bf16", cap)
        assert bp.query() == obucket.plan(numel, eb, cap)
        per = 16384 // eb  # a chunk carries at most 16 KiB
        chunks = sum((n + per - 1) // per for n in numel)
        assert bp.workspace_bytes == 24 * chunks


def test_bucket_slot_addresses_follow_the_oracle_offsets():
    """bucket_plan_slot_address is base + offset * element size, with the
    oracle's next-fit offsets (host arithmetic only: the bucket pointers
    here are fake and never dereferenced)."""
    for numel, dtype, eb in [(configs.c5_numel(), "f32", 4), (configs.c4_numel(), "bf16", 2),
                             ([5, 0, 7, 3, 0], "f32", 4)]:
        bp = gtf.BucketPlan(numel, dtype, configs.BUCKET_CAP_BYTES if len(numel) > 5 else 24)
        bof, off, bn = obucket.plan(numel, eb, configs.BUCKET_CAP_BYTES if len(numel) > 5 else 24)
        bases = [(k + 1) << 32 for k in range(len(bn))]
        arr = C.ptr_array(bases)
        for i in range(len(numel)):
            out = ctypes.c_void_p()
            assert C.lib().bucket_plan_slot_address(bp._h, arr, i, ctypes.byref(out)) == C.GTF_OK
            assert out.value == bases[bof[i]] + off[i] * eb
    bp = gtf.BucketPlan([4, 4], "f32", 16)
    out = ctypes.c_void_p()
    arr = C.ptr_array([1 << 32])
    assert C.lib().bucket_plan_slot_address(bp._h, arr, 2, ctypes.byref(out)) == C.GTF_E_INVALID
    assert C.lib().bucket_plan_slot_address(bp._h, None, 0, ctypes.byref(out)) == C.GTF_E_INVALID
    assert C.lib().bucket_plan_slot_address(bp._h, C.ptr_array([None]), 0,
                                            ctypes.byref(out)) == C.GTF_E_INVALID


def test_multi_set_runs_on_the_host():
    """fuse_multi_*: workspace sized from the items (one per panel of each
    set), a group with a broadcast operand or a reduction refused, run
    before bind refused, a missing pointer refused (no device work)."""
    g = configs.grad_epilogue_graph(1000, avg=configs.AVG_SCALE)
    plan = gtf.FusePlan(g)
    pw = plan.geometry(0)["panel_width"]
    numel = [1000, 0, 8192, 8193, 5, 123457]
    m = gtf.FuseMulti(plan, 0, numel)
    items = sum(-(-n // pw) for n in numel)
    up = lambda x: -(-x // 16) * 16
    nslots = 3
    want = up(up(up(16 * items) + 8 * nslots * len(numel)) + 4 * len(numel))
    assert m.workspace_bytes == want
    assert C.lib().fuse_multi_run(m._h, None) == C.GTF_E_STATE
    ptrs = C.ptr_array([None] * (len(g.tensors) * len(numel)))
    assert C.lib().fuse_multi_bind(m._h, ptrs, ctypes.c_void_p(1 << 20), None) == C.GTF_E_INVALID
    with pytest.raises(gtf.GtfError):
        gtf.FuseMulti(gtf.FusePlan(configs.layernorm_graph(16, 64)), 0, [5])
    with pytest.raises(gtf.GtfError):
        gtf.FuseMulti(gtf.FusePlan(configs.c2_graph(4, 64)), 0, [5])
    with pytest.raises(gtf.GtfError):
        gtf.FuseMulti(plan, 0, [4, -1])


def test_row_resident_plans_match_the_oracle():
    """GTF_ROW_RESIDENT: the library's merged groups equal the oracle's on
    the extension's pinned graphs, the LayerNorm at its c5 size and small
    random DAGs with row reductions, row ops and broadcasts."""
    from tests.test_oracle_partition import _rr_graphs
    graphs = [g for g, _, _ in _rr_graphs().values()]
    graphs.append(configs.layernorm_graph())
    graphs += list(_broadcast_dags(11, 300))
    merged = 0
    for g in graphs:
        plan = gtf.FusePlan(g, row_resident=True)
        want = cap.partition(g, row_resident=True)
        assert as_sets(plan.groups()) == as_sets(want)
        merged += len(want) < len(cap.partition(g))
        for k in range(plan.num_groups):
            geo = plan.geometry(k)
            n_red = sum(g.ops[i].op in ("row_sum", "row_mean", "row_max") for i in plan.group_ops(k))
            # a paired reduction (mean and variance, max and sum of exps) shares a stage
            assert geo["stages"] >= 1 and n_red <= 2 * geo["stages"]
    assert merged >= 20


def test_duplicate_plans_match_the_oracle():
    """GTF_DUPLICATE: the library's rewritten program (op origins) and its
    groups equal the oracle's duplicate() followed by partition(), with and
    without the row-resident merge."""
    from tests.test_oracle_partition import _f32_reduce_dags
    graphs = [configs.layernorm_shared_graph(), configs.layernorm_shared_graph(37, 1000),
              configs.layernorm_graph(), configs.c3_graph(64, 256, head_op=True)]
    graphs += list(_f32_reduce_dags(23, 300)) + list(_broadcast_dags(31, 300))
    changed = 0
    for g in graphs:
        for rr in (False, True):
            plan = gtf.FusePlan(g, row_resident=rr, duplicate=True)
            g2, origin = opart.duplicate(g, row_resident=rr, feasible=cap.group_ok)
            assert plan.op_origin() == origin
            assert plan.n_ops == len(g2.ops)
            assert as_sets(plan.groups()) == as_sets(cap.partition(g2, row_resident=rr))
            changed += g2 is not g
            # internal tensors are never stored: the caller's arrays suffice
            stored = set(plan.materialized())
            want = {t for t in opart.stored_tensors(g2, cap.partition(g2, row_resident=rr))} | \
                set(g.inputs()) | set(g.outputs())
            assert stored == want and max(stored) < len(g.tensors)
    assert changed >= 40


def _lib_bytes_cost(plan):
    """The oracle's bytes_cost, from what the library reports: every tensor
    each launch touches in memory, plus 65536 per launch."""
    b = 0
    for k in range(plan.num_groups):
        for t in plan.group_tensors(k):
            d = plan.graph.tensors[t]
            n = 1
            for e in d.shape:
                n *= e
            b += n * {"f32": 4, "bf16": 2, "u8": 1}[d.dtype]
    return float(b + 65536 * plan.num_groups)


def test_grouped_plans_agree_with_the_oracle_rule():
    """fuse_plan_create_grouped accepts exactly the groupings the oracle's
    plan_ok accepts, on random labelings of random DAGs (most of them
    invalid) and on merges of the fusion pass's groups."""
    from oracle import search as osr
    from tests.test_oracle_partition import _f32_reduce_dags
    rng = np.random.default_rng(77)
    graphs = list(_f32_reduce_dags(61, 150)) + list(_broadcast_dags(62, 150))
    graphs += [configs.layernorm_graph(16, 64), configs.layernorm_shared_graph(16, 64)]
    graphs += list(_gather_dags(60, 150)) + list(_tuple_dags(59, 100))
    n_ok = n_bad = 0
    for g in graphs:
        n = len(g.ops)
        tries = [list(rng.integers(0, max(1, n // 2 + 1), size=n)) for _ in range(6)]
        groups = cap.partition(g)
        for _ in range(3):  # merge two of the fusion pass's groups
            if len(groups) >= 2:
                a, b = rng.choice(len(groups), size=2, replace=False)
                lab = [0] * n
                for k, grp in enumerate(groups):
                    for i in grp:
                        lab[i] = int(a) if k == b else k
                tries.append(lab)
        for lab in tries:
            want = osr.plan_ok(g, [int(x) for x in lab], cap.group_ok)
            try:
                plan = gtf.FusePlan.grouped(g, lab)
                got = True
            except gtf.GtfError as e:
                assert e.status == C.GTF_E_INVALID
                got = False
            assert got == want, (lab, [(o.op, o.inputs, o.output) for o in g.ops])
            if got:
                n_ok += 1
                assert as_sets(plan.groups()) == as_sets(osr.groups_of([int(x) for x in lab]))
            else:
                n_bad += 1
    assert n_ok >= 300 and n_bad >= 300


def test_search_matches_the_oracle():
    """fuse_plan_search with the same seed and the same (byte-count) cost
    follows the oracle's search step for step: the same statistics, the
    same best program and grouping."""
    from oracle import search as osr
    from tests.test_oracle_partition import _f32_reduce_dags
    graphs = [configs.layernorm_shared_graph(16, 64), configs.layernorm_graph(16, 64),
              configs.c3_graph(8, 64, head_op=True), configs.c2_graph(4, 16)]
    graphs += list(_f32_reduce_dags(63, 25)) + list(_broadcast_dags(64, 25)) + list(_gather_dags(65, 25))
    graphs += list(_tuple_dags(66, 25))
    for k, g in enumerate(graphs):
        for seed in (1, 2):
            plan, st = gtf.search(g, _lib_bytes_cost, seed=seed, max_stall=200)
            (prog, origin, lab), ost = osr.search(g, osr.bytes_cost, seed=seed, max_stall=200, feasible=cap.group_ok)
            assert st == ost, (k, seed, st, ost)
            assert plan.op_origin() == origin
            p2 = plan.program()
            assert [(o.op, o.inputs, o.output, np.float32(o.imm)) for o in p2.ops] == \
                [(o.op, o.inputs, o.output, np.float32(o.imm)) for o in prog.ops]
            assert as_sets(plan.groups()) == as_sets(osr.groups_of(lab))


def _gather_dags(seed, count):
    """Small DAGs over [R,C] and [C,R] values (R=3, C=5) with transposes
    between the two, reshapes, concats of [R,C] and [R,2] values, row sums
    and elementwise work."""
    rng = np.random.default_rng(seed)
    R, Cc = 3, 5
    for _ in range(count):
        g = Graph()
        rc = [g.input("x0", "f32", (R, Cc)), g.input("x1", "bf16", (R, Cc))]
        cr = [g.input("y0", "f32", (Cc, R))]
        side = [g.input("w0", "f32", (R, 2))]
        rows = []
        for i in range(int(rng.integers(1, 8))):
            kind = int(rng.integers(0, 8))
            pick = lambda xs: xs[int(rng.integers(len(xs)))]  # noqa: E731
            if kind == 0:
                rc.append(g.op(["exp", "relu", "neg"][int(rng.integers(3))], [pick(rc)], f"t{i}", "f32",
                               (R, Cc)))
            elif kind == 1:
                rc.append(g.op(["add", "mul"][int(rng.integers(2))], [pick(rc), pick(rc)], f"t{i}", "f32",
                               (R, Cc)))
            elif kind == 2:
                rc.append(g.op("transpose", [pick(cr)], f"t{i}", "f32", (R, Cc)))
            elif kind == 3:
                cr.append(g.op("transpose", [pick(rc)], f"t{i}", "f32", (Cc, R)))
            elif kind == 4:
                cr.append(g.op("reshape", [pick(rc)], f"t{i}", "f32", (Cc, R)))
            elif kind == 5:
                cr.append(g.op("neg", [pick(cr)], f"t{i}", "f32", (Cc, R)))
            elif kind == 6:
                a = pick(rc)
                if g.tensors[a].dtype == "f32":
                    c7 = g.op("concat", [a, side[0]], f"t{i}", "f32", (R, Cc + 2))
                    g.op("row_sum", [c7], f"s{i}", "f32", (R, 1), role="out")
            else:
                rows.append(g.op("row_sum", [pick(rc)], f"t{i}", "f32", (R, 1)))
        readers = {t for o in g.ops for t in o.inputs}
        for o in g.ops:
            t = o.output
            if t not in readers or rng.random() < 0.1:
                d = g.tensors[t]
                g.tensors[t] = TensorDesc(d.name, d.dtype, d.shape, "out")
        if g.ops:
            yield g


def test_gather_plans_match_the_oracle():
    """Plans with transposes, reshapes and concats: the library's groups
    equal the oracle's (phase 1 for injective sources; a gathering op only
    as a load), with and without duplicate fusion and the row-resident
    merge."""
    n_fused = 0
    for g in _gather_dags(71, 300):
        for kw in ({}, {"row_resident": True}):
            plan = gtf.FusePlan(g, **kw)
            want = cap.partition(g, **kw)
            assert as_sets(plan.groups()) == as_sets(want), [(o.op, o.inputs, o.output) for o in g.ops]
            n_fused += any(len(grp) > 1 and any(cap.is_gather(g.ops[i]) for i in grp) for grp in want)
        plan = gtf.FusePlan(g, duplicate=True)
        g2, origin = opart.duplicate(g, feasible=cap.group_ok)
        assert plan.op_origin() == origin and as_sets(plan.groups()) == as_sets(cap.partition(g2))
    assert n_fused >= 30


def _tuple_dags(seed, count, R=3, Ca=5, Cb=2):
    """Random graphs around a tuple and the concat of it (TVM's kTuple):
    fields read straight from inputs or made by a transpose, a reshape or an
    element op, moves that change the dtype or whose value is also a graph
    output; the concat stored, scaled, added to a reshaped input, summed per
    row, or the first field of a second tuple."""
    rng = np.random.default_rng(seed)
    for _ in range(count):
        g = Graph()
        dt = ["f32", "bf16"][int(rng.integers(2))]
        other = "bf16" if dt == "f32" else "f32"
        n = [0]

        def name():
            n[0] += 1
            return f"t{n[0]}"

        def field(C):
            k = int(rng.integers(7))
            if k == 0:
                return g.input(name(), dt, (R, C))
            if k in (1, 2):
                return g.op("transpose", [g.input(name(), dt, (C, R))], name(), dt, (R, C))
            if k == 3:
                return g.op("reshape", [g.input(name(), dt, (C, R))], name(), dt, (R, C))
            if k == 4:
                return g.op("exp", [g.input(name(), dt, (R, C))], name(), dt, (R, C))
            if k == 5:   # changes the dtype
                return g.op("transpose", [g.input(name(), other, (C, R))], name(), dt, (R, C))
            return g.op("transpose", [g.input(name(), dt, (C, R))], name(), dt, (R, C), role="out")

        a, b = field(Ca), field(Cb)
        W = Ca + Cb
        c = g.op("concat", [g.op("tuple", [a, b], name(), dt, (R, W))], name(), dt, (R, W))
        k = int(rng.integers(5))
        if k == 0:
            d = g.tensors[c]
            g.tensors[c] = TensorDesc(d.name, d.dtype, d.shape, "out")
        elif k == 1:
            g.op("mul_imm", [c], name(), dt, (R, W), role="out", imm=0.5)
        elif k == 2:
            r = g.op("reshape", [g.input(name(), dt, (W, R))], name(), dt, (R, W))
            g.op("add", [c, r], name(), dt, (R, W), role="out")
        elif k == 3:
            g.op("row_sum", [c], name(), "f32", (R, 1), role="out")
        else:
            e = field(Cb)
            c2 = g.op("concat", [g.op("tuple", [c, e], name(), dt, (R, W + Cb))], name(), dt, (R, W + Cb))
            g.op("neg", [c2], name(), dt, (R, W + Cb), role="out")
        yield g


def test_tuple_plans_match_the_oracle():
    """Plans with tuples: the library's groups equal the oracle's (the tuple
    into its concat in phase 1, its fields into it in phase 2, moves folded
    into the join), with and without the row-resident merge and duplicate
    fusion; in most graphs a move joins its tuple's group."""
    n_phase2 = 0
    for g in _tuple_dags(81, 300):
        for kw in ({}, {"row_resident": True}):
            plan = gtf.FusePlan(g, **kw)
            want = cap.partition(g, **kw)
            assert as_sets(plan.groups()) == as_sets(want), [(o.op, o.inputs, o.output) for o in g.ops]
        tup = [i for i, o in enumerate(g.ops) if o.op == "tuple"]
        n_phase2 += any(g.ops[j].op in ("transpose", "reshape") and
                        any(j in grp and tup[0] in grp for grp in want) for j in range(len(g.ops)))
        plan = gtf.FusePlan(g, duplicate=True)
        g2, origin = opart.duplicate(g, feasible=cap.group_ok)
        assert plan.op_origin() == origin and as_sets(plan.groups()) == as_sets(cap.partition(g2))
    assert n_phase2 >= 100, n_phase2


def test_tuple_and_concat_of_one_operand_errors():
    """A tuple is an intermediate read only by a concat of it alone; a
    concat of one operand reads a tuple and is declared as its shape."""
    a, b = T("a", "f32", (2, 3), "in"), T("b", "f32", (2, 1), "in")
    tup, cat = T("u", "f32", (2, 4), "tmp"), T("c", "f32", (2, 4), "out")
    ok_ops = [OpDesc("tuple", (0, 1), 2), OpDesc("concat", (2,), 3)]
    assert _desc_status([a, b, tup, cat], ok_ops) == C.GTF_OK
    # a tuple as a graph output, or read by another op
    assert _desc_status([a, b, T("u", "f32", (2, 4), "out")], [OpDesc("tuple", (0, 1), 2)]) == C.GTF_E_INVALID
    assert _desc_status([a, b, tup, cat], [OpDesc("tuple", (0, 1), 2), OpDesc("neg", (2,), 3)]) == C.GTF_E_INVALID
    # a concat of one tensor that is not a tuple
    assert _desc_status([T("x", "f32", (2, 4), "in"), cat], [OpDesc("concat", (0,), 1)]) == C.GTF_E_INVALID
    # a concat of a tuple declared at another shape or dtype
    assert _desc_status([a, b, tup, T("c", "f32", (2, 5), "out")], ok_ops) == C.GTF_E_SHAPE
    assert _desc_status([a, b, tup, T("c", "bf16", (2, 4), "out")], ok_ops) == C.GTF_E_SHAPE
    # tuple shapes and dtypes follow concat's
    assert _desc_status([a, T("b", "f32", (3, 1), "in"), tup, cat], ok_ops) == C.GTF_E_SHAPE
    assert _desc_status([a, T("b", "bf16", (2, 1), "in"), tup, cat], ok_ops) == C.GTF_E_UNSUPPORTED
    assert _desc_status([a, b, T("u", "bf16", (2, 4), "tmp"), cat], ok_ops) == C.GTF_E_UNSUPPORTED


def test_new_entry_point_errors():
    """Error behaviour of the grouped-plan, search and program entry points
    and of the data-movement ops' shape checks (host only)."""
    L = C.lib()
    x = T("x", "f32", (2, 3), "in")
    # transpose / reshape / concat shapes
    assert _desc_status([x, T("t", "f32", (3, 2), "out")], [OpDesc("transpose", (0,), 1)]) == C.GTF_OK
    assert _desc_status([x, T("t", "f32", (2, 3), "out")], [OpDesc("transpose", (0,), 1)]) == C.GTF_E_SHAPE
    assert _desc_status([T("v", "f32", (6,), "in"), T("t", "f32", (6, 1), "out")],
                        [OpDesc("transpose", (0,), 1)]) == C.GTF_E_SHAPE   # rank 1
    assert _desc_status([x, T("r", "f32", (6,), "out")], [OpDesc("reshape", (0,), 1)]) == C.GTF_OK
    assert _desc_status([x, T("r", "f32", (7,), "out")], [OpDesc("reshape", (0,), 1)]) == C.GTF_E_SHAPE
    z = T("z", "f32", (2, 4), "in")
    assert _desc_status([x, z, T("c", "f32", (2, 7), "out")], [OpDesc("concat", (0, 1), 2)]) == C.GTF_OK
    assert _desc_status([x, z, T("c", "f32", (2, 8), "out")], [OpDesc("concat", (0, 1), 2)]) == C.GTF_E_SHAPE
    assert _desc_status([x, T("w", "f32", (3, 4), "in"), T("c", "f32", (2, 7), "out")],
                        [OpDesc("concat", (0, 1), 2)]) == C.GTF_E_SHAPE   # row counts differ
    assert _desc_status([x, T("w", "bf16", (2, 4), "in"), T("c", "f32", (2, 7), "out")],
                        [OpDesc("concat", (0, 1), 2)]) == C.GTF_E_UNSUPPORTED   # two dtypes
    # grouped plans: a cycle, a negative label, NULL labels
    g = Graph()
    a = g.input("a", "f32", (4, 8))
    b = g.op("exp", [a], "b", "f32", (4, 8))
    c = g.op("neg", [b], "c", "f32", (4, 8))
    g.op("relu", [c], "d", "f32", (4, 8), role="out")
    assert gtf.FusePlan.grouped(g, [0, 0, 0]).num_groups == 1
    for lab in ([0, 1, 0], [0, -1, 0]):
        with pytest.raises(gtf.GtfError) as e:
            gtf.FusePlan.grouped(g, lab)
        assert e.value.status == C.GTF_E_INVALID
    desc, tens, ops = gtf._program_desc(g)
    h = ctypes.c_void_p()
    assert L.fuse_plan_create_grouped(ctypes.byref(desc), None, ctypes.byref(h)) == C.GTF_E_INVALID
    assert h.value is None
    assert L.fuse_plan_create_grouped(ctypes.byref(desc), None, None) == C.GTF_E_INVALID
    # search: bad parameters, a failing cost, an exception in the cost
    with pytest.raises(gtf.GtfError) as e:
        gtf.search(g, lambda p: 1.0, alpha=0.5)
    assert e.value.status == C.GTF_E_INVALID
    with pytest.raises(gtf.GtfError) as e:
        gtf.search(g, lambda p: -1.0)
    assert e.value.status == C.GTF_E_INVALID and b"cost" in L.gtf_last_error()
    with pytest.raises(ZeroDivisionError):
        gtf.search(g, lambda p: 1 / 0)
    # the search's plan is the best it costed: a cost that prefers fewer
    # launches ends with one group
    best, st = gtf.search(g, lambda p: float(p.num_groups), max_stall=50)
    assert best.num_groups == 1 and st["best_cost"] == 1.0 and st["start_cost"] == 3.0
    # program: capacities
    plan = gtf.FusePlan(g)
    nt, no = ctypes.c_int32(), ctypes.c_int32()
    assert L.fuse_plan_program(plan._h, None, 0, ctypes.byref(nt), None, 0, ctypes.byref(no)) == 0
    assert (nt.value, no.value) == (4, 3)
    small = (C.TensorDesc * 1)()
    assert L.fuse_plan_program(plan._h, small, 1, None, None, 0, None) == C.GTF_E_LIMIT
    assert plan.program().ops == g.ops
    # group tensors: capacity and index
    n = ctypes.c_int32()
    assert L.fuse_plan_group_tensors(plan._h, 5, None, 0, ctypes.byref(n)) == C.GTF_E_INVALID
    assert L.fuse_plan_group_tensors(plan._h, 0, None, 0, ctypes.byref(n)) == 0 and n.value == 2
    one = (ctypes.c_int32 * 1)()
    assert L.fuse_plan_group_tensors(plan._h, 0, one, 1, ctypes.byref(n)) == C.GTF_E_LIMIT


def test_binding_refuses_host_tensors_before_any_launch():
    """The binding checks every torch tensor it marshals (on the GPU,
    contiguous, the plan's exact size): a host tensor is refused with
    ValueError before the library is called."""
    import torch
    g = configs.gelu_graph(4, 8)
    plan = gtf.FusePlan(g)
    host = {t: torch.zeros(g.tensors[t].shape, dtype=torch.int16) for t in range(len(g.tensors))}
    with pytest.raises(ValueError, match="not a GPU tensor"):
        plan.run(host)
    bp = gtf.BucketPlan([10, 20], "f32", 1 << 20)
    with pytest.raises(ValueError, match="not a GPU tensor"):
        bp.pack([torch.zeros(10), torch.zeros(20)], [torch.zeros(30)], 0.5)
    with pytest.raises(ValueError, match="1 tensors for a plan of 2"):
        bp.pack([torch.zeros(10)], [torch.zeros(30)], 0.5)


def test_binding_refuses_short_pointer_lists_before_any_launch():
    """A list of tensors shorter than the graph, or fewer tensor sets than a
    multi-set run was created for, would make the library read past the
    pointer array: the binding refuses both with ValueError before the
    library is called."""
    import torch
    g = configs.gelu_graph(4, 8)
    plan = gtf.FusePlan(g)
    short = [torch.zeros(g.tensors[t].shape, dtype=torch.int16) for t in range(len(g.tensors) - 1)]
    with pytest.raises(ValueError, match=f"{len(short)} tensors for a graph of {len(g.tensors)}"):
        plan.run(short)
    with pytest.raises(ValueError, match="tensors for a graph of"):
        plan.launcher(0, short)
    ge = configs.grad_epilogue_graph(16)
    pe = gtf.FusePlan(ge)
    multi = gtf.FuseMulti(pe, 0, [16, 16, 16])
    with pytest.raises(ValueError, match="2 tensor sets for a run of 3"):
        multi.bind([{}, {}], torch.zeros(16, dtype=torch.uint8))
