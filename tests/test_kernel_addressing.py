"""Host-side replay of the executor's tile walk (no GPU): for every group of
the workloads and of the edge shapes the GPU tests run, each lane's tiles
and each ring prefetch address must stay inside the tensors they read.

The replay restates the element loop of the executor kernel: items are
(row block, column panel); 256 threads split into rows of threads_per_row
lanes; lane tiles q = (pass, j); a prefetch for a tile that is not a whole
in-range tile falls back to the tensor's first tile."""
import numpy as np
import pytest

import gradient_tensor_fusion_amd as gtf
from workloads import configs
from workloads.graph import Graph

KV, BLOCK = 8, 256


def _numel(graph, t):
    n = 1
    for s in graph.tensors[t].shape:
        n *= s
    return n


def replay(graph, plan, g):
    geo = plan.geometry(g)
    R, C = geo["rows"], geo["cols"]
    tpr, RB, PW = geo["threads_per_row"], geo["rows_per_item"], geo["panel_width"]
    panels, items = geo["panels"], geo["items"]
    assert PW % KV == 0 and BLOCK % tpr == 0 and items == -(-R // RB) * panels or R == 0
    rpp = BLOCK // tpr
    erow = 0 if R == 1 else C
    tid = np.arange(BLOCK)
    sub, lt = tid // tpr, tid % tpr
    ring_numel = [_numel(graph, t) for t in geo["ring_tensor"]]
    if geo["ring_inputs"]:
        assert geo["ring_stages"] >= 2 and C >= KV and geo["lds_bytes"] <= 64 * 1024
        assert all(n >= KV for n in ring_numel)
    n_tiles = 0
    for item in range(items):
        rb, p = divmod(item, panels)
        r0, c0 = rb * RB, p * PW
        nr, nc = min(RB, R - r0), min(PW, C - c0)
        assert nr > 0 and nc >= 0
        npass = -(-nr // rpp)
        tpl = max(1, -(-nc // (tpr * KV)))
        q = np.arange(npass * tpl)
        rr = (q // tpl)[None, :] * rpp + sub[:, None]
        cl = (lt[:, None] + (q % tpl)[None, :] * tpr) * KV
        ok = (rr < nr) & (cl + KV <= nc)
        eoff = np.where(ok, (r0 + rr) * erow + c0 + cl, 0)
        for n in ring_numel:
            assert np.all(eoff >= 0) and np.all(eoff + KV <= n), (item, n)
        valid = (rr < nr) & (cl < nc)
        cnt = np.minimum(KV, nc - cl)
        last = (r0 + rr) * erow + c0 + cl + cnt - 1
        assert np.all(last[valid] < R * C)
        # each tile of the item exactly once
        ids = (rr * (nc // KV + 1) + cl // KV)[valid]
        assert ids.size == np.unique(ids).size == nr * (-(-nc // KV))
        n_tiles += int(valid.sum())
    want = R * sum(-(-min(PW, C - p * PW) // KV) for p in range(panels)) if C > 0 else 0
    assert n_tiles == want


def cases():
    out = []
    for sh in [(64, 512), (3, 5), (2, 67), (1, 1), (130, 24)]:
        out.append(("c1", configs.c1_graph(*sh)))
    for sh in [(4096, 4096), (64, 1000), (33, 1024), (2, 67), (1, 9), (5, 130), (0, 8), (4, 0), (0, 0),
               (16, 1024)]:
        out.append(("c2", configs.c2_graph(*sh)))
    for sh, h in [((8192, 4096), False), ((8192, 4096), True), ((40, 1000), False), ((3, 5), True),
                  ((2, 67), False), ((5, 130), False), ((4, 65536), False), ((7, 8), False),
                  ((64, 4096), False), ((512, 4096), False), ((4, 0), False)]:
        out.append(("c3", configs.c3_graph(*sh, head_op=h)))
    for sh in [(8192, 1024), (37, 1024), (16, 264), (3, 5), (64, 1024)]:
        out.append(("ln", configs.layernorm_graph(*sh)))
    for sh in [(8192, 4096), (9, 4096), (5, 130), (2, 67), (64, 4096)]:
        out.append(("gelu", configs.gelu_graph(*sh)))
    for sh in [(8192, 1024), (11, 1000), (2, 67), (64, 1024)]:
        out.append(("drop", configs.dropout_graph(*sh)))
    g = Graph()
    x = g.input("x", "f32", (64, 1024))
    for op in ("exp", "tanh", "sigmoid", "gelu"):
        g.op(op, [x], op, "f32", (64, 1024), role="out")
    out.append(("transc", g))
    return out


@pytest.mark.parametrize("name,graph", cases())
def test_tile_walk_and_ring_stay_in_bounds(name, graph):
    for fuse in (True, False):
        plan = gtf.FusePlan(graph, fuse=fuse)
        for g in range(plan.num_groups):
            replay(graph, plan, g)


def test_random_dag_shapes_stay_in_bounds():
    from tests.test_capi_host import _broadcast_dags
    from tests.test_gpu_parity import _reshape
    from tests.test_oracle_partition import _random_dags
    for gen in (_random_dags(31, 40, 4), _broadcast_dags(7, 60)):
        for g in gen:
            for R, C in [(1, 1), (3, 5), (2, 67), (5, 130), (1, 9)]:
                gg = _reshape(g, R, C)
                for fuse in (True, False):
                    plan = gtf.FusePlan(gg, fuse=fuse)
                    for k in range(plan.num_groups):
                        replay(gg, plan, k)
