"""The allocation-free pack (bucket_pack_static) against bucket_pack: two
calls in a row on one GPU, the second with a smaller plan (fewer chunks
than the table the first call left in the library's static array), bit
for bit against bucket_pack on the same inputs and against the oracle's
pack; and a chunk table over the array's 1 MiB refused before any launch."""
import ctypes

import numpy as np
import pytest
import torch

import gradient_tensor_fusion_amd as gtf
from gradient_tensor_fusion_amd import _capi as C
from oracle import bucket as obucket
from tests.gpu_util import announce, assert_bits_equal, to_device
from workloads import configs

pytestmark = pytest.mark.gpu


def _buckets(bn):
    return [torch.full((n,), float("nan"), dtype=torch.float32, device="cuda") for n in bn]


@pytest.mark.parametrize("order", ["large_then_small", "small_then_large"])
def test_pack_static_matches_bucket_pack_on_two_calls(order):
    cases = [(configs.c4_numel(), 4101, configs.BUCKET_CAP_BYTES),
             ([5, 1000, 0, 77777, 3, 16385], 4102, 1 << 18)]
    if order == "small_then_large":
        cases = cases[::-1]
    for numel, seed, cap in cases:
        announce("bucket_pack_static", order, len(numel), "tensors", sum(numel), "elements")
        host = configs.gradient_values(numel, seed)
        dev = [to_device(h, "f32") for h in host]
        bp = gtf.BucketPlan(numel, "f32", cap)
        _, _, bn = bp.query()
        ws = torch.empty(max(16, bp.workspace_bytes), dtype=torch.uint8, device="cuda")
        bp.bind(ws)
        want = _buckets(bn)
        bp.pack(dev, want, configs.AVG_SCALE)
        got = _buckets(bn)
        # straight through the C ABI
        st = C.lib().bucket_pack_static(bp._h, bp._tensor_ptrs(dev), bp._bucket_ptrs(got),
                                        ctypes.c_float(configs.AVG_SCALE), None)
        assert st == C.GTF_OK, C.lib().gtf_last_error()
        torch.cuda.synchronize()
        for g, w in zip(got, want):
            assert_bits_equal(g.cpu().numpy(), w.cpu().numpy())
        ref = obucket.pack(numel, 4, cap, host, configs.AVG_SCALE)
        for g, r in zip(got, ref):
            assert_bits_equal(g.cpu().numpy(), np.asarray(r, dtype=np.float32))


def test_pack_static_refuses_a_table_over_its_array():
    """50,000 one-element tensors make 50,000 chunks (1.2 MB of table): the
    call fails with GTF_E_LIMIT before anything is copied or launched."""
    n = 50000
    one = torch.zeros(1, dtype=torch.float32, device="cuda")
    bp = gtf.BucketPlan([1] * n, "f32", 1 << 30)
    _, _, bn = bp.query()
    bucket = torch.zeros(bn[0], dtype=torch.float32, device="cuda")
    src = C.ptr_array([one.data_ptr()] * n)
    st = C.lib().bucket_pack_static(bp._h, src, C.ptr_array([bucket.data_ptr()]),
                                    ctypes.c_float(1.0), None)
    assert st == C.GTF_E_LIMIT
    assert b"static scratch" in C.lib().gtf_last_error()
    torch.cuda.synchronize()
    assert torch.all(bucket == 0)
