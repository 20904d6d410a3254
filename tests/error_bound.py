"""Per-element error bounds for comparing a fused run with the oracle
(test infrastructure: it reads the oracle's values, never the HIP path).

The stated bars fix what the library may differ by, op by op:
  * IEEE basic ops (add, sub, mul, div, sqrt, max, min, square, recip, neg,
    relu, the immediate forms, add3, dmul, copy and the data movements) are
    correctly rounded on both sides: given identical operands the results
    are identical, so they add no error of their own -- only, once their
    operands already differ, the propagated difference and one fp32 ulp per
    rounding that may land on the other side (add3, (a + b) + c, rounds
    twice: one ulp of a + b and one of the result);
  * exp, tanh, sigmoid and gelu add at most 1e-6 of the oracle's value (the
    elementwise fp32 bar), plus a few units of fp32's smallest subnormal,
    where 1e-6 of a subnormal is below the format's resolution;
  * row sums and means add at most 1e-5 of the sum of the magnitudes of the
    reduced terms (the reduction bar, read against the terms' magnitudes,
    which stays meaningful where they cancel); row max adds nothing;
  * a value stored as bf16 may round to the neighbouring bf16 value once
    its fp32 value differs at all.
Differences propagate through each op by a bound on its derivative over
the interval the operand may lie in, doubled for second-order effects.
Where the bound is 0 the outputs must be bit-identical (+0 and -0 aside)."""
from __future__ import annotations

import numpy as np

from oracle import evaluate as oev
from oracle import numerics
from oracle import partition as opart

TRANSCENDENTAL = ("exp", "tanh", "sigmoid", "gelu")
REDUCES = ("row_sum", "row_mean", "row_max")
REL = 1e-6           # elementwise fp32 bar
RED = 1e-5           # reduction bar
TINY = 4 * 2.0 ** -149


def _ulp32(v):
    a = np.abs(np.asarray(v, dtype=np.float64))
    a = np.where(np.isfinite(a), a, 0.0)
    return np.spacing(a.astype(np.float32)).astype(np.float64)


def _ulp_bf16(v):
    a = np.abs(np.asarray(v, dtype=np.float64))
    a = np.where(np.isfinite(a), a, 0.0)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -133)))
    return np.where(a >= 2.0 ** -126, 2.0 ** (e - 7), 2.0 ** -133)


def _sigmoid_d(z):
    # sigmoid'(z) = e / (1 + e)^2 with e = exp(-|z|): no 1 - s, which is 0
    # in float64 from |z| ~ 37 on while the derivative is still ~1e-16 there
    # and, against sigmoid's own tiny tail values, far from negligible
    e = np.exp(-np.abs(z))
    return e / (1.0 + e) ** 2


def _propagate(op, a, b, imm, out_shape):
    """Bound on |f(x~) - f(x)| from the operands' values a and bounds b (first
    order over the interval, doubled)."""
    with np.errstate(all="ignore"):
        if op in ("copy", "neg", "relu", "add_imm"):
            p = b[0]
        elif op in ("add", "sub", "max", "min"):
            p = b[0] + b[1]
        elif op == "add3":
            p = b[0] + b[1] + b[2]
        elif op == "mul_imm":
            p = abs(np.float32(imm)) * b[0]
        elif op == "dmul":
            p = abs(np.float32(imm)) * np.abs(a[1]) * b[0]
        elif op == "mul":
            p = np.abs(a[1]) * b[0] + np.abs(a[0]) * b[1] + b[0] * b[1]
        elif op == "square":
            p = 2 * np.abs(a[0]) * b[0] + b[0] * b[0]
        elif op in ("div", "recip"):
            num, den = (a[0], a[1]) if op == "div" else (1.0, a[0])
            bn, bd = (b[0], b[1]) if op == "div" else (0.0, b[0])
            lo = np.abs(den) - bd
            p = np.where(lo > 0, bn / np.maximum(lo, 1e-300) + np.abs(num) * bd /
                         np.maximum(np.abs(den) * lo, 1e-300), np.inf)
        elif op == "sqrt":
            x = np.maximum(a[0], 0.0)
            p = np.minimum(b[0] / np.maximum(np.sqrt(x) + np.sqrt(np.maximum(x - b[0], 0.0)), 1e-300),
                           np.sqrt(b[0]))
        elif op == "exp":
            p = np.exp(a[0]) * np.expm1(b[0])
        elif op == "tanh":
            near0 = np.maximum(np.abs(a[0]) - b[0], 0.0)
            p = (1.0 - np.tanh(near0) ** 2) * b[0]
        elif op == "sigmoid":
            near0 = np.maximum(np.abs(a[0]) - b[0], 0.0)
            p = _sigmoid_d(near0) * b[0]
        elif op == "gelu":
            p = 1.13 * b[0]        # |GELU'| <= 1.13 everywhere
        elif op == "transpose":
            p = np.asarray(b[0]).T
        elif op in ("reshape",):
            p = np.broadcast_to(b[0], a[0].shape).reshape(out_shape)
        elif op in ("concat", "tuple"):
            p = np.concatenate([np.broadcast_to(b[k], a[k].shape) for k in range(len(a))], axis=1)
        else:
            raise ValueError(op)
    return 2.0 * np.broadcast_to(p, out_shape)


def run_with_bounds(graph, inputs, groups):
    """The oracle's evaluation of the graph under this grouping, with a
    bound for every tensor: (stored values, {tensor: bound on the stored
    value})."""
    stored = opart.stored_tensors(graph, groups)
    raw = {}
    vals = oev.evaluate(graph, inputs, stored, groups=groups, raw_out=raw)
    group_of = {i: k for k, grp in enumerate(groups) for i in grp}
    producer = {o.output: i for i, o in enumerate(graph.ops)}
    b_raw, b_st = {}, {}
    for t in graph.inputs():
        b_raw[t] = b_st[t] = np.zeros(vals[t].shape)
    for j, o in enumerate(graph.ops):
        a, b = [], []
        for t in o.inputs:
            same = producer.get(t) is not None and group_of.get(producer[t]) == group_of.get(j)
            a.append(np.asarray(raw[t] if same else vals[t], dtype=np.float64))
            b.append(b_raw[t] if same else b_st[t])
        out = np.asarray(raw[o.output], dtype=np.float64)
        with np.errstate(all="ignore"):
            if o.op in REDUCES:
                terms = a[0]
                if o.op == "row_max":
                    e = b[0].max(axis=-1, keepdims=True) if terms.shape[-1] else np.zeros(out.shape)
                else:
                    mag = np.abs(terms).sum(axis=-1, keepdims=True)
                    e = np.broadcast_to(b[0], terms.shape).sum(axis=-1, keepdims=True) + RED * np.maximum(
                        mag, np.abs(terms.sum(axis=-1, keepdims=True)))
                    if o.op == "row_mean":
                        e = e / max(terms.shape[-1], 1)
                    e = e + _ulp32(out)
            else:
                prop = _propagate(o.op, a, b, o.imm, out.shape)
                if o.op in TRANSCENDENTAL:
                    e = prop + REL * (np.abs(out) + prop) + TINY
                else:
                    r = _ulp32(out)
                    if o.op == "add3":   # (a + b) is rounded before c is added
                        r = r + _ulp32(np.abs(a[0]) + np.abs(a[1]))
                    e = prop + np.where(prop > 0, r, 0.0)
        e = np.where(np.isfinite(out), np.asarray(e, dtype=np.float64), 0.0)
        b_raw[o.output] = e
        d = graph.tensors[o.output]
        if d.dtype == "bf16" and (o.output in stored or d.role == "out"):
            b_st[o.output] = e + np.where(e > 0, _ulp_bf16(vals[o.output]), 0.0)
        else:
            b_st[o.output] = e
    return vals, b_st


def assert_within(got, want_vals, bound, dtype, what=""):
    """|got - want| <= bound element by element (decoded to fp32 values);
    equal where the bound is 0 (zeros of either sign equal), both NaN or
    equal infinities accepted."""
    g = np.asarray(numerics.decode(np.asarray(got).reshape(want_vals.shape), dtype), dtype=np.float64)
    w = np.asarray(want_vals, dtype=np.float64)
    bnd = np.broadcast_to(bound, w.shape)
    same = (g == w) | (np.isnan(g) & np.isnan(w))
    with np.errstate(invalid="ignore"):   # inf - inf where both are the same infinity
        err = np.where(same, 0.0, np.abs(g - w))
    bad = ~(err <= bnd)
    if bad.any():
        i = tuple(int(k) for k in np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} elements outside the bound; "
                             f"first at {i}: got {g[i]!r} want {w[i]!r} bound {bnd[i]!r}")
    return float((err / np.where(bnd > 0, bnd, 1.0)).max()) if err.size else 0.0
