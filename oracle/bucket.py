"""Tensor-fusion buckets (oracle, test infrastructure only).

DisCo (arXiv 2209.12769) section 1: tensor fusion joins small gradient
tensors into one fused tensor before the AllReduce, and the fused tensor's
size is the sum of the members' sizes; the AllReduce sums or averages the
gradients.  Section 7 and the AllReduce-combiner passage describe the
threshold rule (Horovod's fusion threshold, XLA's combiner): neighbouring
tensors are combined while the fused size stays within a threshold.

Planning here is next-fit in the given (production) order: tensor i joins
the open bucket when bucket_bytes + bytes_i <= cap, or when the open bucket
is still empty; otherwise a new bucket opens with tensor i.  So a tensor
larger than the cap sits alone.  Offsets are dense prefix sums inside each
bucket (no padding, no splitting).  A zero-size tensor takes the current
offset of the open bucket.

pack:   bucket[b][off_i + j] = fl32(src_i[j] * s)
unpack: dst_i[j]             = fl32(bucket[b][off_i + j] * s)
with s the fp32 value of the scale; s == 1 copies the bits unchanged.
The averaging reading puts s = 1/N on the pack side.
"""
from __future__ import annotations

from typing import List, Sequence, Tuple

import numpy as np


def plan(numel: Sequence[int], elem_bytes: int, cap_bytes: int
         ) -> Tuple[List[int], List[int], List[int]]:
    """(bucket_of, offset, bucket_numel), offsets in elements."""
    bucket_of: List[int] = []
    offset: List[int] = []
    bucket_numel: List[int] = []
    for n in numel:
        nbytes = int(n) * elem_bytes
        if bucket_numel:
            fill = bucket_numel[-1] * elem_bytes
            fits = fill + nbytes <= cap_bytes or fill == 0
        else:
            fits = False
        if not fits:
            bucket_numel.append(0)
        bucket_of.append(len(bucket_numel) - 1)
        offset.append(bucket_numel[-1])
        bucket_numel[-1] += int(n)
    return bucket_of, offset, bucket_numel


def _scaled(x: np.ndarray, scale: float) -> np.ndarray:
    s = np.float32(scale)
    x = np.asarray(x, dtype=np.float32)
    if s == np.float32(1.0):
        return x.copy()
    with np.errstate(all="ignore"):
        return (x * s).astype(np.float32)


def pack(numel, elem_bytes, cap_bytes, srcs: List[np.ndarray], scale: float
         ) -> List[np.ndarray]:
    bucket_of, offset, bucket_numel = plan(numel, elem_bytes, cap_bytes)
    buckets = [np.zeros(n, dtype=np.float32) for n in bucket_numel]
    for i, x in enumerate(srcs):
        n = int(numel[i])
        buckets[bucket_of[i]][offset[i]:offset[i] + n] = _scaled(x.reshape(-1), scale)
    return buckets


def unpack(numel, elem_bytes, cap_bytes, buckets: List[np.ndarray], scale: float
           ) -> List[np.ndarray]:
    bucket_of, offset, _ = plan(numel, elem_bytes, cap_bytes)
    out = []
    for i, n in enumerate(numel):
        n = int(n)
        out.append(_scaled(buckets[bucket_of[i]][offset[i]:offset[i] + n], scale))
    return out
