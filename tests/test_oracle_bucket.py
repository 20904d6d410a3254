"""Pins for the oracle's tensor-fusion buckets (DisCo section 1: fused size is
the sum of member sizes; threshold-bounded combining)."""
import json
import os

import numpy as np

from oracle import bucket
from workloads import configs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_hand_worked_plans():
    with open(os.path.join(GOLDEN, "bucket_small.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        b, o, n = bucket.plan(c["numel"], c["elem_bytes"], c["cap_bytes"])
        assert (b, o, n) == (c["bucket_of"], c["offset"], c["bucket_numel"]), c


def _check_plan_properties(numel, eb, cap):
    b, o, n = bucket.plan(numel, eb, cap)
    # sizes add up: every element has exactly one place
    assert sum(n) == sum(numel)
    # production order is kept
    assert all(b[i] <= b[i + 1] for i in range(len(b) - 1))
    # each bucket is tiled exactly, no gap, no overlap
    for k in range(len(n)):
        members = [i for i in range(len(numel)) if b[i] == k]
        pos = 0
        for i in members:
            assert o[i] == pos
            pos += numel[i]
        assert pos == n[k]
        # within the cap, unless the bucket is a lone oversize tensor
        big = [i for i in members if numel[i] * eb > cap]
        assert n[k] * eb <= cap or (len([i for i in members if numel[i] > 0]) == 1 and big)
    # next-fit: the first non-empty tensor of a bucket would not have fit
    # in the bucket before it
    for k in range(1, len(n)):
        first = next(i for i in range(len(numel)) if b[i] == k)
        assert n[k - 1] * eb + numel[first] * eb > cap and n[k - 1] > 0


def test_plan_properties_on_random_lists():
    rng = np.random.default_rng(5)
    for _ in range(300):
        cnt = int(rng.integers(0, 40))
        numel = [int(v) for v in rng.integers(0, 50, size=cnt)]
        numel = [0 if rng.random() < 0.1 else v for v in numel]
        cap = int(rng.integers(1, 200)) * 4
        _check_plan_properties(numel, 4, cap)


def test_c4_and_c5_plans():
    for numel in (configs.c4_numel(), configs.c5_numel()):
        _check_plan_properties(numel, 4, configs.BUCKET_CAP_BYTES)
    _, _, n4 = bucket.plan(configs.c4_numel(), 4, configs.BUCKET_CAP_BYTES)
    _, _, n5 = bucket.plan(configs.c5_numel(), 4, configs.BUCKET_CAP_BYTES)
    assert len(n4) >= 4 and len(n5) >= 24


def _special_f32():
    bits = np.array([0x7FC00001, 0xFFC12345, 0x7F800000, 0xFF800000, 0x80000000,
                     0x00000001, 0x807FFFFF, 0x3F800000], dtype=np.uint32)
    return bits.view(np.float32)


def test_pack_then_unpack_with_scale_one_is_the_identity_bitwise():
    numel = [5, 0, 17, 3, 64, 1]
    srcs = [configs.gradient_values(numel, 9)[i] for i in range(len(numel))]
    srcs[2][:8] = _special_f32()
    bks = bucket.pack(numel, 4, 40, srcs, 1.0)
    back = bucket.unpack(numel, 4, 40, bks, 1.0)
    for a, b in zip(srcs, back):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_power_of_two_scales_are_exact():
    numel = [100, 7, 1000]
    srcs = configs.gradient_values(numel, 10)
    bks = bucket.pack(numel, 4, 1024, srcs, 0.125)
    for i, x in enumerate(srcs):
        b, o, _ = bucket.plan(numel, 4, 1024)
        seg = bks[b[i]][o[i]:o[i] + numel[i]]
        assert np.array_equal(seg * np.float32(8.0), x)      # exact both ways
    back = bucket.unpack(numel, 4, 1024, bks, 8.0)
    for a, c in zip(srcs, back):
        assert np.array_equal(a, c)


def test_pack_places_each_tensor_at_its_offset():
    numel = [3, 5, 2, 7]
    srcs = [np.arange(n, dtype=np.float32) + 10 * i for i, n in enumerate(numel)]
    bks = bucket.pack(numel, 4, 32, srcs, 1.0)
    assert bks[0].tolist() == [0, 1, 2, 10, 11, 12, 13, 14]
    assert bks[1].tolist() == [20, 21]
    assert bks[2].tolist() == list(range(30, 37))


def test_joint_epilogue_equals_separate_pack():
    """Folding the 1/N average into a gradient epilogue (joint op and tensor
    fusion) gives the same bucket bits as running the epilogue and packing
    with scale 1/N: scaling by a power of two is exact for normal values,
    so the one multiply lands on the same float either way."""
    from oracle import evaluate as oev
    numel = [1000, 37, 4096, 5, 0, 333]
    joint, sep = [], []
    for k, n in enumerate(numel):
        gj = configs.grad_epilogue_graph(n, avg=configs.AVG_SCALE)
        gs = configs.grad_epilogue_graph(n)
        inp = configs.grad_epilogue_inputs(gj, k)
        oj = oev.outputs(gj, oev.evaluate(gj, inp))[gj.outputs()[0]]
        # same input ids in both graphs: g and w are the first two tensors
        os_ = oev.outputs(gs, oev.evaluate(gs, inp))[gs.outputs()[0]]
        joint.append(np.asarray(oj, dtype=np.float32).reshape(-1))
        sep.append(np.asarray(os_, dtype=np.float32).reshape(-1))
        assert np.all(np.abs(sep[-1][sep[-1] != 0]) > 1e-30)
    cap = 4 * 2048
    a = bucket.pack(numel, 4, cap, joint, 1.0)
    b = bucket.pack(numel, 4, cap, sep, configs.AVG_SCALE)
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))
