"""Helpers for the GPU parity tests: device buffers from the seeded host
arrays, running a graph through the C ABI, and the comparators."""
from __future__ import annotations

import sys
from typing import Dict

import numpy as np
import torch

import gradient_tensor_fusion_amd as gtf
from tests import capacity as cap
from oracle import evaluate as oev
from oracle import numerics
from oracle import partition as opart

TORCH_DT = {"f32": torch.float32, "bf16": torch.int16, "u8": torch.uint8}


def announce(*what) -> None:
    print("[gpu case]", *what, file=sys.stderr, flush=True)


def to_device(arr: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).cuda()
    if dtype == "u8":
        return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.uint8)).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).cuda()


def to_host(t: torch.Tensor, dtype: str) -> np.ndarray:
    a = t.cpu().numpy()
    if dtype == "bf16":
        return a.view(np.uint16)
    return a


def empty_device(shape, dtype: str) -> torch.Tensor:
    return torch.empty(tuple(shape), dtype=TORCH_DT[dtype], device="cuda")


def gpu_run(graph, inputs: Dict[int, np.ndarray], fuse: bool = True, plan=None,
            row_resident: bool = False):
    """Run the graph on the GPU; returns (plan, {tensor id: host array}) for
    every materialised tensor (bf16 as uint16 bits)."""
    plan = plan or gtf.FusePlan(graph, fuse=fuse, row_resident=row_resident)
    dev = {}
    for t in plan.materialized():
        d = graph.tensors[t]
        if d.role == "in":
            dev[t] = to_device(inputs[t], d.dtype)
        else:
            dev[t] = empty_device(d.shape, d.dtype)
            if d.dtype == "f32":
                dev[t].fill_(float("nan"))
            else:
                dev[t].fill_(0x7FC1 if d.dtype == "bf16" else 0)
    plan.run(dev)
    torch.cuda.synchronize()
    host = {t: to_host(v, graph.tensors[t].dtype) for t, v in dev.items()}
    return plan, host


def oracle_run(graph, inputs, fuse: bool = True, given=None, row_resident: bool = False):
    groups = cap.partition(graph, fuse=fuse, row_resident=row_resident)
    stored = opart.stored_tensors(graph, groups)
    return oev.run(graph, inputs, stored=stored, given=given, groups=groups)


def bf16_ulps(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    def ordered(x):
        x = np.asarray(x, dtype=np.uint16).astype(np.int32)
        mag = x & 0x7FFF
        return np.where(x & 0x8000, -mag, mag)
    return np.abs(ordered(a) - ordered(b))


def assert_bf16_close(got, want, max_ulp=1):
    got = np.asarray(got).view(np.uint16).ravel()
    want = np.asarray(want).view(np.uint16).ravel()
    gn = np.isnan(numerics.bf16_to_f32(got))
    wn = np.isnan(numerics.bf16_to_f32(want))
    assert np.array_equal(gn, wn), "NaN pattern differs"
    d = bf16_ulps(got[~gn], want[~gn])
    worst = int(d.max()) if d.size else 0
    assert worst <= max_ulp, f"bf16 max ulp distance {worst} > {max_ulp} ({int((d > max_ulp).sum())} elements)"
    return worst


def assert_f32_rel(got, want, rel):
    got = np.asarray(got, dtype=np.float32).ravel().astype(np.float64)
    want = np.asarray(want, dtype=np.float32).ravel().astype(np.float64)
    both_nan = np.isnan(got) & np.isnan(want)
    zero = want == 0
    assert np.all(got[zero & ~both_nan] == 0), "expected exact zeros"
    nz = ~zero & ~both_nan
    err = np.abs(got[nz] - want[nz]) / np.abs(want[nz])
    worst = float(err.max()) if err.size else 0.0
    assert worst <= rel, f"max relative error {worst:.3e} > {rel:.1e}"
    return worst


def assert_bits_equal(got, want):
    g = np.ascontiguousarray(got)
    w = np.ascontiguousarray(want)
    assert g.shape == w.shape and g.dtype.itemsize == w.dtype.itemsize, (g.shape, w.shape)
    u = "u%d" % g.dtype.itemsize
    gi, wi = g.view(u).ravel(), w.view(u).ravel()
    diff = np.nonzero(gi != wi)[0]
    if diff.size:
        i = int(diff[0])
        raise AssertionError(f"{diff.size} of {gi.size} elements differ; first at {i}: "
                             f"got {g.ravel()[i]!r} ({int(gi[i]):#x}) want {w.ravel()[i]!r} ({int(wi[i]):#x})")


def reduce_bound(vals_in: np.ndarray, mean: bool) -> np.ndarray:
    """Sum of magnitudes of the reduced terms per row (fp64): the scale the
    reduction tolerance is relative to."""
    s = np.abs(vals_in.astype(np.float64)).sum(axis=-1)
    if mean:
        s = s / vals_in.shape[-1]
    return s


def assert_reduce_close(got, want, scale, rel=1e-5):
    got = np.asarray(got, dtype=np.float32).ravel().astype(np.float64)
    want = np.asarray(want, dtype=np.float32).ravel().astype(np.float64)
    scale = np.asarray(scale, dtype=np.float64).ravel()
    err = np.abs(got - want)
    lim = rel * np.maximum(scale, np.abs(want))
    worst = float((err / np.maximum(lim / rel, 1e-300)).max()) if err.size else 0.0
    assert np.all(err <= lim), f"reduction error {worst:.3e} of magnitude sum > {rel:.0e}"
    return worst


def assert_close_scaled(got, want, rel, scale):
    """|got - want| <= rel * (|want| + scale): for graphs whose
    transcendental or reduced values pass through additions, where a tiny
    relative error of an operand is measured against the operand size."""
    g = np.asarray(got, dtype=np.float64).ravel()
    w = np.asarray(want, dtype=np.float64).ravel()
    both_nan = np.isnan(g) & np.isnan(w)
    err = np.abs(g - w)[~both_nan]
    lim = rel * (np.abs(w[~both_nan]) + scale)
    worst = float((err / lim).max()) if err.size else 0.0
    assert np.all(err <= lim), f"error {worst:.2f} x the scaled tolerance {rel:.0e}"
    return worst
