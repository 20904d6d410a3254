"""Sizes past 2^31 elements on the GPU, checked on sampled outputs.

Index arithmetic is 64-bit throughout the executor and the bucket kernel;
these cases put elements on both sides of 2^31 and at the ragged end, and
compare samples (the first, the last, those around 2^31 and random ones)
with the oracle's evaluation of the same values.  Inputs follow the pattern
v(i) = ((i mod 255) - 127) / 8, exact in bf16, whose row sums are exact in
fp32, so every comparison is bit for bit."""
import numpy as np
import pytest
import torch

import gradient_tensor_fusion_amd as gtf
from oracle import bucket as obucket
from oracle import evaluate as oev
from oracle import numerics
from tests.gpu_util import announce, assert_bits_equal
from workloads import configs
from workloads.graph import Graph

pytestmark = pytest.mark.gpu

BIG = (1 << 31) + 8003          # elements: past 2^31, with a ragged tail
CHUNK = 1 << 27


def _pattern_host(idx):
    return (((idx % 255) - 127) / 8.0).astype(np.float32)


def _fill_pattern(t, start=0):
    """t (1-D, on the GPU) <- v(start + i), chunk by chunk."""
    n = t.numel()
    for c0 in range(0, n, CHUNK):
        c1 = min(n, c0 + CHUNK)
        i = torch.arange(start + c0, start + c1, device="cuda", dtype=torch.int64)
        t[c0:c1] = ((i % 255) - 127).to(torch.float32).div_(8.0).to(t.dtype)
        del i


def _samples(n, rng, k=1024):
    around = np.arange((1 << 31) - k, (1 << 31) + k, dtype=np.int64)
    idx = np.concatenate([np.arange(k), np.arange(n - k, n), around[around < n],
                          rng.integers(0, n, size=k)])
    return np.unique(idx)


def test_flat_elementwise_past_2_31_elements():
    announce("large flat", BIG)
    g = Graph()
    x = g.input("x", "bf16", (BIG,))
    g.op("mul_imm", [x], "y", "bf16", (BIG,), role="out", imm=2.0)
    plan = gtf.FusePlan(g)
    assert plan.num_groups == 1
    xd = torch.empty(BIG, dtype=torch.bfloat16, device="cuda")
    _fill_pattern(xd)
    yd = torch.empty(BIG, dtype=torch.bfloat16, device="cuda")
    plan.run({0: xd.view(torch.int16), 1: yd.view(torch.int16)})
    torch.cuda.synchronize()
    idx = _samples(BIG, np.random.default_rng(1))
    got = yd.view(torch.int16)[torch.from_numpy(idx).cuda()].cpu().numpy().view(np.uint16)
    # the oracle on the sampled inputs, as one row
    gs = Graph()
    xs = gs.input("x", "bf16", (1, idx.size))
    gs.op("mul_imm", [xs], "y", "bf16", (1, idx.size), role="out", imm=2.0)
    xin = configs.to_bf16_bits(_pattern_host(idx).astype(np.float64)).reshape(1, -1)
    _, want = oev.run(gs, {xs: xin})
    assert_bits_equal(got, want[1].ravel())
    del xd, yd
    torch.cuda.empty_cache()


def test_row_sum_past_2_31_elements():
    R, C = (1 << 21) + 7, 1024          # 2^31 + 7168 elements
    announce("large row sum", R, C)
    g = Graph()
    X = g.input("X", "bf16", (R, C))
    g.op("row_sum", [X], "s", "f32", (R, 1), role="out")
    plan = gtf.FusePlan(g)
    xd = torch.empty(R * C, dtype=torch.bfloat16, device="cuda")
    _fill_pattern(xd)
    sd = torch.empty(R, dtype=torch.float32, device="cuda")
    plan.run({0: xd.view(torch.int16).view(R, C), 1: sd.view(R, 1)})
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(64), np.arange(R - 64, R),
                                     np.arange((1 << 21) - 64, (1 << 21) + 7),
                                     np.random.default_rng(2).integers(0, R, size=256)]))
    got = sd[torch.from_numpy(rows).cuda()].cpu().numpy()
    gs = Graph()
    Xs = gs.input("X", "bf16", (rows.size, C))
    gs.op("row_sum", [Xs], "s", "f32", (rows.size, 1), role="out")
    el = (rows[:, None].astype(np.int64) * C + np.arange(C)[None, :])
    xin = configs.to_bf16_bits(_pattern_host(el).astype(np.float64))
    _, want = oev.run(gs, {Xs: xin})
    assert_bits_equal(got, want[1].ravel())
    del xd, sd
    torch.cuda.empty_cache()


def test_bucket_pack_unpack_past_2_31_elements():
    numel = [1000, (1 << 31) + 5, 7]
    announce("large buckets", numel)
    cap = configs.BUCKET_CAP_BYTES
    bof, off, bn = obucket.plan(numel, 4, cap)
    bp = gtf.BucketPlan(numel, "f32", cap)
    assert [list(v) for v in bp.query()] == [bof, off, bn]
    ws = torch.empty(max(16, bp.workspace_bytes), dtype=torch.uint8, device="cuda")
    bp.bind(ws)
    starts = np.concatenate([[0], np.cumsum(numel)[:-1]]).astype(np.int64)
    src = []
    for n, s0 in zip(numel, starts):
        t = torch.empty(n, dtype=torch.float32, device="cuda")
        _fill_pattern(t, int(s0))
        src.append(t)
    buckets = [torch.empty(n, dtype=torch.float32, device="cuda") for n in bn]
    bp.pack(src, buckets, configs.AVG_SCALE)
    back = [torch.empty(n, dtype=torch.float32, device="cuda") for n in numel]
    bp.unpack(buckets, back, 1.0)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    for i, (n, s0) in enumerate(zip(numel, starts)):
        idx = _samples(n, rng, 256) if n > 4096 else np.arange(n)
        vals = _pattern_host(s0 + idx)
        want = obucket._scaled(vals, configs.AVG_SCALE)
        b = buckets[bof[i]][torch.from_numpy(off[i] + idx).cuda()].cpu().numpy()
        assert_bits_equal(b, want)
        assert_bits_equal(back[i][torch.from_numpy(idx).cuda()].cpu().numpy(), want)
    del src, buckets, back
    torch.cuda.empty_cache()
