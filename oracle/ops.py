"""What each op computes (oracle, test infrastructure only).

Every op takes fp32 operands and gives an fp32 result:

* add, sub, mul, div, max, min, square (x*x), sqrt, recip (1/x), neg,
  add_imm, mul_imm, add3 ((a+b)+c), dmul ((h*s)*mask) and copy are IEEE
  binary32 operations, each correctly rounded to nearest-even; NumPy float32
  arithmetic is exactly that.
* relu(x) is x when x > 0 and +0.0 otherwise.
* exp, tanh, sigmoid(z) = 1/(1+e^-z) and gelu(z) = z/2 * erfc(-z/sqrt(2))
  (the exact-erf GELU written with erfc so that its negative tail keeps its
  relative accuracy) are evaluated in float64 and rounded once to fp32.
* row_sum / row_mean reduce the last axis: float64 accumulation of the fp32
  values, then one rounding to fp32; the mean divides the float64 sum by
  the row width before that rounding.
* row_max is the largest value of each row (exact; -inf for an empty row,
  the identity of max).  Sum, mean and max are the commutative reductions
  of TVM "Operator Pattern Classification" (kCommReduce).

Operands broadcast NumPy-style over two axes ([R,C], [1,C], [R,1], [1,1]).
Op fusion does not change what a graph computes; it only keeps the
intermediates on chip (DisCo section 1; TVM "Operator Fusion", FuseTIR).
So this per-op table, applied one op at a time, is the definition the fused
kernels are checked against.
"""
from __future__ import annotations

import numpy as np
from scipy.special import erfc

F32 = np.float32


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _imm(v: float) -> np.float32:
    return F32(v)


def exp(x):
    return np.exp(_f64(x)).astype(F32)


def tanh(x):
    return np.tanh(_f64(x)).astype(F32)


def sigmoid(x):
    z = _f64(x)
    return (1.0 / (1.0 + np.exp(-z))).astype(F32)


def gelu(x):
    z = _f64(x)
    return (0.5 * z * erfc(-z / np.sqrt(2.0))).astype(F32)


def relu(x):
    x = np.asarray(x, dtype=F32)
    return np.where(x > F32(0), x, F32(0)).astype(F32)


def row_sum(x):
    x = np.asarray(x, dtype=F32)
    return _f64(x).sum(axis=-1, keepdims=True).astype(F32)


def row_mean(x):
    x = np.asarray(x, dtype=F32)
    return (_f64(x).sum(axis=-1, keepdims=True) / x.shape[-1]).astype(F32)


def row_max(x):
    x = np.asarray(x, dtype=F32)
    if x.shape[-1] == 0:
        return np.full(x.shape[:-1] + (1,), -np.inf, dtype=F32)
    return x.max(axis=-1, keepdims=True).astype(F32)


def apply(op: str, args, imm: float = 0.0, shape=None) -> np.ndarray:
    """One op on fp32 arrays (2-D [R, C]); shape is the result's shape,
    needed by reshape."""
    a = [np.asarray(v, dtype=F32) for v in args]
    with np.errstate(all="ignore"):
        if op == "copy":
            r = a[0].copy()
        elif op == "transpose":
            r = a[0].T.copy()
        elif op == "reshape":
            r = a[0].reshape(shape).copy()   # row-major element order kept
        elif op == "tuple":
            # a tuple's fields, held as one [R, C1 + C2] value whose only
            # reader is the concat of that tuple
            r = np.concatenate([a[0], a[1]], axis=1)
        elif op == "concat":
            r = np.concatenate(a, axis=1)   # two tensors, or the one tuple
        elif op == "exp":
            r = exp(a[0])
        elif op == "tanh":
            r = tanh(a[0])
        elif op == "sigmoid":
            r = sigmoid(a[0])
        elif op == "relu":
            r = relu(a[0])
        elif op == "gelu":
            r = gelu(a[0])
        elif op == "square":
            r = a[0] * a[0]
        elif op == "sqrt":
            r = np.sqrt(a[0])
        elif op == "recip":
            r = F32(1.0) / a[0]
        elif op == "neg":
            r = -a[0]
        elif op == "add_imm":
            r = a[0] + _imm(imm)
        elif op == "mul_imm":
            r = a[0] * _imm(imm)
        elif op == "add":
            r = a[0] + a[1]
        elif op == "sub":
            r = a[0] - a[1]
        elif op == "mul":
            r = a[0] * a[1]
        elif op == "div":
            r = a[0] / a[1]
        elif op == "max":
            r = np.maximum(a[0], a[1])
        elif op == "min":
            r = np.minimum(a[0], a[1])
        elif op == "add3":
            r = (a[0] + a[1]) + a[2]
        elif op == "dmul":
            r = (a[0] * _imm(imm)) * a[1]
        elif op == "row_sum":
            r = row_sum(a[0])
        elif op == "row_mean":
            r = row_mean(a[0])
        elif op == "row_max":
            r = row_max(a[0])
        else:
            raise ValueError(f"unknown op {op}")
    return np.asarray(r, dtype=F32)
