"""Host-side replay of the executor's tile walk (no GPU): for every group of
the workloads and of the edge shapes the GPU tests run, every element a lane
loads or stores must lie inside the tensors, and every 8-element tile of the
domain must be visited exactly once.

The replay restates the element loop of the executor kernel: items are
(row block, column panel); 256 threads split into rows of threads_per_row
(tpr) lanes; a lane's tiles are runs of K sub-tiles of 8 elements, tpr * 8
elements apart in its row.  A run whose K sub-tiles are whole in all 64
lanes of a wave goes to the whole-tile interpreter at once (16-byte accesses
for tensors aligned for them, else one access per element); otherwise each
sub-tile is handled on its own, partial ones element by element."""
import numpy as np
import pytest

import gradient_tensor_fusion_amd as gtf
from workloads import configs
from workloads.graph import Graph

KV, BLOCK, WAVE = 8, 256, 64


def replay(graph, plan, g):
    geo = plan.geometry(g)
    R, C = geo["rows"], geo["cols"]
    tpr, RB, PW = geo["threads_per_row"], geo["rows_per_item"], geo["panel_width"]
    panels, items, K = geo["panels"], geo["items"], geo["subtiles"]
    assert K in (1, 4) and geo["spill_slots"] <= geo["spill_slots_max"]
    assert geo["spill_slots_max"] in ((0, 2) if K == 4 else (6,))
    assert PW % KV == 0 and BLOCK % tpr == 0 and (items == -(-R // RB) * panels or R == 0)
    assert geo["lds_bytes"] <= 64 * 1024
    rpp = BLOCK // tpr
    ks = tpr * KV
    erow = 0 if R == 1 else C
    vec_ok = R == 1 or C % KV == 0
    numel = R * C
    tid = np.arange(BLOCK)
    sub, lt = tid // tpr, tid % tpr
    seen = []
    for item in range(items):
        rb, p = divmod(item, panels)
        r0, c0 = rb * RB, p * PW
        nr, nc = min(RB, R - r0), min(PW, C - c0)
        assert nr > 0 and nc >= 0
        npass = -(-nr // rpp)
        tpl = max(1, -(-nc // ks))
        spl = -(-tpl // K)
        for q in range(npass * spl):
            ps, s = divmod(q, spl)
            rr = ps * rpp + sub
            cl0 = (lt + s * K * tpr) * KV
            whole = (rr < nr) & (cl0 + (K - 1) * ks + KV <= nc)
            fast = np.repeat(whole.reshape(-1, WAVE).all(axis=1), WAVE)
            for k in range(K):
                cl = cl0 + k * ks
                valid = (rr < nr) & (cl < nc)
                cnt = np.where(fast, KV, np.clip(nc - cl, 0, KV))
                first = (r0 + rr) * erow + c0 + cl
                on = valid | fast
                assert np.all(fast <= valid)
                assert np.all(first[on] >= 0) and np.all(first[on] + cnt[on] <= numel), (item, q, k)
                # whole sub-tiles of tensors whose rows are a multiple of 8
                # take 16-byte accesses: they start on a multiple of 8
                if vec_ok:
                    assert np.all(first[fast] % KV == 0)
                seen.append((r0 + rr)[on] * (C // KV + 1) + (c0 + cl)[on] // KV)
    want = R * sum(-(-min(PW, C - p * PW) // KV) for p in range(panels)) if C > 0 else 0
    ids = np.concatenate(seen) if seen else np.zeros(0, dtype=np.int64)
    assert ids.size == np.unique(ids).size == want


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
    for sh in [(131072, 128), (37, 1000), (5, 4097), (3, 5)]:
        out.append(("softmax", configs.softmax_graph(*sh)))
    g = Graph()
    x = g.input("x", "f32", (64, 1024))
    for op in ("exp", "tanh", "sigmoid", "gelu"):
        g.op(op, [x], op, "f32", (64, 1024), role="out")
    out.append(("transc", g))
    return out


@pytest.mark.parametrize("name,graph", cases())
def test_tile_walk_stays_in_bounds(name, graph):
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
