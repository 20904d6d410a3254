"""Op-by-op, unfused evaluation of a graph (oracle, test infrastructure only).

Each op runs on its own, in the graph's (topological) order, and every
intermediate is kept as an fp32 array.  Two things decide where values get
rounded to a narrower type:

* graph outputs are stored in their declared dtype;
* a tensor listed in ``stored`` (an intermediate that crosses from one fused
  group to another, or every intermediate when nothing is fused) is written
  to memory in its declared dtype and read back, so later ops see the
  rounded value.

Inside a fused group the intermediates never leave the chip (DisCo section
1; TVM "Operator Fusion", FuseTIR), so they stay fp32; that is the only
difference between a fused and an unfused run.
"""
from __future__ import annotations

from typing import Dict, Iterable, Tuple

import numpy as np

from . import numerics, ops


def norm_shape(shape: Tuple[int, ...]) -> Tuple[int, int]:
    """Rank-1 [N] is the row vector [1, N]; rank 2 is kept."""
    if len(shape) == 1:
        return (1, int(shape[0]))
    if len(shape) == 2:
        return (int(shape[0]), int(shape[1]))
    raise ValueError(f"rank {len(shape)} not supported")


def _extent(ns) -> int:
    """NumPy rule for one axis: extents of 1 stretch to the others (also to 0)."""
    other = {n for n in ns if n != 1}
    if len(other) > 1:
        raise ValueError(f"extents {ns} do not broadcast")
    return other.pop() if other else 1


def broadcast_shape(shapes) -> Tuple[int, int]:
    R = _extent([s[0] for s in shapes])
    C = _extent([s[1] for s in shapes])
    for r, c in shapes:
        if r not in (1, R) or c not in (1, C):
            raise ValueError(f"shapes {shapes} do not broadcast")
    return (R, C)


def result_shape(op: str, in_shapes, declared=None) -> Tuple[int, int]:
    if op in ("row_sum", "row_mean", "row_max"):
        return (in_shapes[0][0], 1)
    if op == "transpose":
        return (in_shapes[0][1], in_shapes[0][0])
    if op == "reshape":
        # the declared shape, provided the element count is kept
        if declared[0] * declared[1] != in_shapes[0][0] * in_shapes[0][1]:
            raise ValueError(f"reshape of {in_shapes[0]} to {declared}")
        return declared
    if op == "concat" and len(in_shapes) == 1:   # the concat of one tuple
        return in_shapes[0]
    if op in ("concat", "tuple"):
        (r1, c1), (r2, c2) = in_shapes
        if r1 != r2:
            raise ValueError(f"concat of {in_shapes}: row counts differ")
        return (r1, c1 + c2)
    return broadcast_shape(in_shapes)


def evaluate(graph, inputs: Dict[int, np.ndarray],
             stored: Iterable[int] = (), given: Dict[int, np.ndarray] = None,
             groups=None, raw_out: Dict[int, np.ndarray] = None) -> Dict[int, np.ndarray]:
    """fp32 value of every tensor as it is in memory (rounded to its dtype
    where it is stored: graph outputs and ``stored`` intermediates), each
    shaped [R, C].

    ``given`` maps tensor ids to fp32 values used instead of computing them
    (their producing ops are skipped): a later group can then be checked on
    exactly the inputs another implementation handed it.

    ``groups`` (lists of op indices): an op reading a value produced in its
    own group gets the value before the store's rounding, since inside a
    fused group every intermediate is fp32 and rounding happens only at the
    store (TVM "FuseTIR": the group is one function whose intermediates
    never go through memory).  Without groups, every reader of a stored
    value gets the rounded value (each op its own group).
    ``raw_out``, when given, receives each op's fp32 result before any
    store rounding (what readers in the producer's own group see).
    """
    stored = set(stored)
    given = {} if given is None else given
    group_of = {}
    for k, grp in enumerate(groups or []):
        for i in grp:
            group_of[i] = k
    producer = {o.output: i for i, o in enumerate(graph.ops)}
    raw: Dict[int, np.ndarray] = {}
    vals: Dict[int, np.ndarray] = {}
    for t in graph.inputs():
        d = graph.tensors[t]
        vals[t] = numerics.decode(inputs[t], d.dtype).reshape(norm_shape(d.shape))
    for j, o in enumerate(graph.ops):
        if o.output in given:
            d = graph.tensors[o.output]
            vals[o.output] = np.asarray(given[o.output], dtype=np.float32).reshape(norm_shape(d.shape))
            raw[o.output] = vals[o.output]
            continue
        args = []
        for i in o.inputs:
            p = producer.get(i)
            same = p is not None and groups is not None and group_of.get(p) == group_of.get(j)
            args.append(raw[i] if same else vals[i])
        d = graph.tensors[o.output]
        want = result_shape(o.op, [a.shape for a in args], norm_shape(d.shape))
        if norm_shape(d.shape) != want:
            raise ValueError(f"{o.op} -> {d.name}: declared {d.shape}, computes {want}")
        r = ops.apply(o.op, args, o.imm, want)
        r = np.broadcast_to(r, want).astype(np.float32)
        raw[o.output] = r
        if o.output in stored or d.role == "out":
            r = numerics.round_to(r, d.dtype)
        vals[o.output] = r
    if raw_out is not None:
        raw_out.update(raw)
    return vals


def outputs(graph, vals: Dict[int, np.ndarray]) -> Dict[int, np.ndarray]:
    """Graph outputs encoded in their declared dtype (bf16 as uint16 bits),
    in the declared shape."""
    res = {}
    for t in graph.outputs():
        d = graph.tensors[t]
        res[t] = numerics.encode(vals[t], d.dtype).reshape(d.shape)
    return res


def run(graph, inputs: Dict[int, np.ndarray], stored: Iterable[int] = (), given=None,
        groups=None):
    """Convenience: evaluate and return (all fp32 values, encoded outputs)."""
    vals = evaluate(graph, inputs, stored, given, groups)
    return vals, outputs(graph, vals)
