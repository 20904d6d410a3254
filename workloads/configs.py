"""The five synthetic workloads: their op graphs and their seeded inputs.

Inputs are drawn in float64 from ``workloads.rng``, rounded to float32, and,
for bf16 tensors, rounded once more to bfloat16 by round-to-nearest-even
(PyTorch's CPU conversion).  bf16 tensors are returned as uint16 bit
patterns, u8 tensors as uint8, f32 tensors as float32.

c1  RNNLM-style chain, f32[64,512]:   y = sigmoid((x*a)*b)
c2  broadcast group, bf16[4096,4096]: out = relu(X + bias) + R
c3  diamond + row reduce, bf16[8192,4096] -> f32[8192,1]:
        s = rowsum((exp(P) + 0.5*P) + tanh(P))
c4  161 fp32 gradient tensors (frozen sizes), N(0, 1e-3), 25 MiB buckets, 1/8
c5  12 layers of Transformer-block groups over 8192 tokens x 1024 hidden:
        LayerNorm (mean, variance, normalise), bias + GELU on [8192,4096],
        dropout (keep 0.9) + residual; plus 194 fp32 gradient tensors.

joint  op and tensor fusion together: each of c5's 194 parameter gradients
       goes through an elementwise epilogue g' = g * (1/loss_scale) + wd * w
       (loss-scale removal and weight decay), and the epilogue's store puts
       g' * (1/N) straight into the gradient's bucket slot.

Every builder takes the sizes as arguments so tests can run the same graph
at small shapes.
"""
from __future__ import annotations

from typing import Dict, List, Tuple

import numpy as np
import torch

from . import rng, sizes
from .graph import Graph

BUCKET_CAP_BYTES = 25 * 1024 * 1024
AVG_SCALE = 1.0 / 8.0          # data-parallel average over 8 replicas
LN_EPS = 1e-5
DROP_P = 0.1


def to_bf16_bits(x64: np.ndarray) -> np.ndarray:
    f32 = torch.from_numpy(np.ascontiguousarray(x64, dtype=np.float64).astype(np.float32))
    return f32.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def _f32(x64: np.ndarray) -> np.ndarray:
    return x64.astype(np.float32)


def _draw(kind: str, seed: int, stream: int, n: int, a: float, b: float) -> np.ndarray:
    if kind == "uniform":
        return rng.uniform(seed, stream, n, a, b)
    return rng.normal(seed, stream, n, a, b)


def tensor_values(dtype: str, shape, kind: str, seed: int, stream: int,
                  a: float, b: float) -> np.ndarray:
    n = int(np.prod(shape))
    x = _draw(kind, seed, stream, n, a, b).reshape(shape)
    if dtype == "bf16":
        return to_bf16_bits(x)
    return _f32(x)


# ---------------------------------------------------------------- c1
def c1_graph(rows: int = 64, cols: int = 512) -> Graph:
    g = Graph()
    x = g.input("x", "f32", (rows, cols))
    a = g.input("a", "f32", (rows, cols))
    b = g.input("b", "f32", (rows, cols))
    m1 = g.op("mul", [x, a], "mul1", "f32", (rows, cols))
    m2 = g.op("mul", [m1, b], "mul2", "f32", (rows, cols))
    g.op("sigmoid", [m2], "y", "f32", (rows, cols), role="out")
    return g


def c1_inputs(g: Graph, seed: int = 1) -> Dict[int, np.ndarray]:
    return {t: tensor_values("f32", g.tensors[t].shape, "uniform", seed, s, -1.0, 1.0)
            for s, t in enumerate(g.inputs())}


# ---------------------------------------------------------------- c2
def c2_graph(rows: int = 4096, cols: int = 4096) -> Graph:
    g = Graph()
    X = g.input("X", "bf16", (rows, cols))
    bias = g.input("bias", "bf16", (cols,))
    R = g.input("R", "bf16", (rows, cols))
    t1 = g.op("add", [X, bias], "bias_add", "bf16", (rows, cols))
    t2 = g.op("relu", [t1], "relu", "bf16", (rows, cols))
    g.op("add", [t2, R], "out", "bf16", (rows, cols), role="out")
    return g


def c2_inputs(g: Graph, seed: int = 2) -> Dict[int, np.ndarray]:
    X, bias, R = g.inputs()
    sh = g.tensors
    return {X: tensor_values("bf16", sh[X].shape, "normal", seed, 0, 0.0, 1.0),
            bias: tensor_values("bf16", sh[bias].shape, "normal", seed, 1, 0.0, 0.1),
            R: tensor_values("bf16", sh[R].shape, "normal", seed, 2, 0.0, 1.0)}


# ---------------------------------------------------------------- c3
def c3_graph(rows: int = 8192, cols: int = 4096, head_op: bool = False) -> Graph:
    """Diamond: P feeds exp, 0.5*P and tanh, which meet in one 3-input add,
    then a row sum.  With head_op the diamond's head is an op (P*1) instead
    of the graph input, so the post-dominator of an op decides the group."""
    g = Graph()
    P = g.input("P", "bf16", (rows, cols))
    if head_op:
        P = g.op("mul_imm", [P], "head", "bf16", (rows, cols), imm=1.0)
    e = g.op("exp", [P], "exp", "bf16", (rows, cols))
    h = g.op("mul_imm", [P], "half", "bf16", (rows, cols), imm=0.5)
    t = g.op("tanh", [P], "tanh", "bf16", (rows, cols))
    s = g.op("add3", [e, h, t], "add3", "bf16", (rows, cols))
    g.op("row_sum", [s], "rowsum", "f32", (rows, 1), role="out")
    return g


def c3_inputs(g: Graph, seed: int = 3) -> Dict[int, np.ndarray]:
    (P,) = g.inputs()
    return {P: tensor_values("bf16", g.tensors[P].shape, "uniform", seed, 0, -2.0, 2.0)}


# ---------------------------------------------------------------- c5 groups
def layernorm_graph(rows: int = 8192, hidden: int = 1024, eps: float = LN_EPS) -> Graph:
    """LayerNorm written op by op.  x - mean appears twice (once for the
    variance, once for the normalised output), so neither later group needs
    a stored x - mean."""
    g = Graph()
    X = g.input("X", "bf16", (rows, hidden))
    gamma = g.input("gamma", "bf16", (hidden,))
    beta = g.input("beta", "bf16", (hidden,))
    mean = g.op("row_mean", [X], "mean", "f32", (rows, 1))
    d1 = g.op("sub", [X, mean], "xc_var", "bf16", (rows, hidden))
    sq = g.op("square", [d1], "sq", "bf16", (rows, hidden))
    var = g.op("row_mean", [sq], "var", "f32", (rows, 1))
    d2 = g.op("sub", [X, mean], "xc_out", "bf16", (rows, hidden))
    ve = g.op("add_imm", [var], "var_eps", "f32", (rows, 1), imm=eps)
    sd = g.op("sqrt", [ve], "std", "f32", (rows, 1))
    rs = g.op("recip", [sd], "rstd", "f32", (rows, 1))
    nrm = g.op("mul", [d2, rs], "norm", "bf16", (rows, hidden))
    sc = g.op("mul", [nrm, gamma], "scaled", "bf16", (rows, hidden))
    g.op("add", [sc, beta], "y", "bf16", (rows, hidden), role="out")
    return g


def layernorm_shared_graph(rows: int = 8192, hidden: int = 1024, eps: float = LN_EPS) -> Graph:
    """The same LayerNorm with x - mean written once and read twice (by the
    square and by the normalisation): what duplicate fusion starts from."""
    g = Graph()
    X = g.input("X", "bf16", (rows, hidden))
    gamma = g.input("gamma", "bf16", (hidden,))
    beta = g.input("beta", "bf16", (hidden,))
    mean = g.op("row_mean", [X], "mean", "f32", (rows, 1))
    xc = g.op("sub", [X, mean], "xc", "bf16", (rows, hidden))
    sq = g.op("square", [xc], "sq", "bf16", (rows, hidden))
    var = g.op("row_mean", [sq], "var", "f32", (rows, 1))
    ve = g.op("add_imm", [var], "var_eps", "f32", (rows, 1), imm=eps)
    sd = g.op("sqrt", [ve], "std", "f32", (rows, 1))
    rs = g.op("recip", [sd], "rstd", "f32", (rows, 1))
    nrm = g.op("mul", [xc, rs], "norm", "bf16", (rows, hidden))
    sc = g.op("mul", [nrm, gamma], "scaled", "bf16", (rows, hidden))
    g.op("add", [sc, beta], "y", "bf16", (rows, hidden), role="out")
    return g


def softmax_graph(rows: int = 131072, cols: int = 128) -> Graph:
    """Row softmax written op by op, the way a framework writes it for
    numerical range: y = exp(x - max x) * (1 / sum exp(x - max x)).  The
    default shape is the attention probabilities of 8192 tokens cut into 64
    sequences of 128 with 16 heads.  exp(x - max) appears twice (once for
    the sum, once for the output), so neither later group needs it stored."""
    g = Graph()
    X = g.input("X", "bf16", (rows, cols))
    m = g.op("row_max", [X], "max", "f32", (rows, 1))
    d1 = g.op("sub", [X, m], "xm_sum", "bf16", (rows, cols))
    e1 = g.op("exp", [d1], "e_sum", "bf16", (rows, cols))
    s = g.op("row_sum", [e1], "sum", "f32", (rows, 1))
    d2 = g.op("sub", [X, m], "xm_out", "bf16", (rows, cols))
    e2 = g.op("exp", [d2], "e_out", "bf16", (rows, cols))
    r = g.op("recip", [s], "rsum", "f32", (rows, 1))
    g.op("mul", [e2, r], "y", "bf16", (rows, cols), role="out")
    return g


def softmax_inputs(g: Graph, seed: int) -> Dict[int, np.ndarray]:
    (X,) = g.inputs()
    return {X: tensor_values("bf16", g.tensors[X].shape, "normal", seed, 5, 0.0, 2.0)}


def gelu_graph(rows: int = 8192, ffn: int = 4096) -> Graph:
    g = Graph()
    A = g.input("A", "bf16", (rows, ffn))
    b = g.input("b1", "bf16", (ffn,))
    t = g.op("add", [A, b], "bias_add", "bf16", (rows, ffn))
    g.op("gelu", [t], "y", "bf16", (rows, ffn), role="out")
    return g


def dropout_graph(rows: int = 8192, hidden: int = 1024, p: float = DROP_P) -> Graph:
    g = Graph()
    h = g.input("h", "bf16", (rows, hidden))
    m = g.input("mask", "u8", (rows, hidden))
    R = g.input("R", "bf16", (rows, hidden))
    keep_scale = float(np.float32(1.0 / (1.0 - p)))
    d = g.op("dmul", [h, m], "dropped", "bf16", (rows, hidden), imm=keep_scale)
    g.op("add", [d, R], "y", "bf16", (rows, hidden), role="out")
    return g


def layernorm_inputs(g: Graph, seed: int) -> Dict[int, np.ndarray]:
    X, gamma, beta = g.inputs()
    sh = g.tensors
    return {X: tensor_values("bf16", sh[X].shape, "normal", seed, 0, 0.0, 1.0),
            gamma: tensor_values("bf16", sh[gamma].shape, "normal", seed, 1, 1.0, 0.1),
            beta: tensor_values("bf16", sh[beta].shape, "normal", seed, 2, 0.0, 0.1)}


def gelu_inputs(g: Graph, seed: int) -> Dict[int, np.ndarray]:
    A, b = g.inputs()
    sh = g.tensors
    return {A: tensor_values("bf16", sh[A].shape, "normal", seed, 3, 0.0, 1.0),
            b: tensor_values("bf16", sh[b].shape, "normal", seed, 4, 0.0, 0.1)}


def dropout_inputs(g: Graph, seed: int, p: float = DROP_P) -> Dict[int, np.ndarray]:
    h, m, R = g.inputs()
    sh = g.tensors
    n = int(np.prod(sh[m].shape))
    keep = (rng.uniform(seed, 6, n) >= p).astype(np.uint8).reshape(sh[m].shape)
    return {h: tensor_values("bf16", sh[h].shape, "normal", seed, 5, 0.0, 1.0),
            m: keep,
            R: tensor_values("bf16", sh[R].shape, "normal", seed, 7, 0.0, 1.0)}


def c5_layer_seed(layer: int) -> int:
    return 5000 + layer


LOSS_SCALE_INV = 1.0 / 1024.0  # exact in fp32
WEIGHT_DECAY = 0.01
JOINT_SEED = 5200


def grad_epilogue_graph(n: int, avg=None, inv_scale: float = LOSS_SCALE_INV,
                        wd: float = WEIGHT_DECAY) -> Graph:
    """g' = g * inv_scale + wd * w over one fp32 gradient of n elements;
    with avg, the output is g' * avg (the data-parallel average folded into
    the epilogue, whose output then lives in a bucket slot)."""
    g = Graph()
    gr = g.input("g", "f32", (n,))
    w = g.input("w", "f32", (n,))
    a = g.op("mul_imm", [gr], "g_unscaled", "f32", (n,), imm=inv_scale)
    b = g.op("mul_imm", [w], "decay", "f32", (n,), imm=wd)
    if avg is None:
        g.op("add", [a, b], "g_out", "f32", (n,), role="out")
    else:
        c = g.op("add", [a, b], "g_sum", "f32", (n,))
        g.op("mul_imm", [c], "g_avg", "f32", (n,), role="out", imm=avg)
    return g


def grad_epilogue_inputs(g: Graph, index: int, seed: int = JOINT_SEED) -> Dict[int, np.ndarray]:
    """Loss-scaled gradient ~ N(0, 1) and weights ~ N(0, 0.02), two streams
    per tensor index."""
    gr, w = g.inputs()
    n = int(np.prod(g.tensors[gr].shape))
    return {gr: _f32(rng.normal(seed, 2 * index, n, 0.0, 1.0)),
            w: _f32(rng.normal(seed, 2 * index + 1, n, 0.0, 0.02))}


# ---------------------------------------------------------------- buckets
def gradient_values(numel: List[int], seed: int, std: float = 1e-3,
                    which=None) -> List[np.ndarray]:
    """fp32 gradients ~ N(0, std), one counter stream per tensor."""
    idx = range(len(numel)) if which is None else which
    return [_f32(rng.normal(seed, i, numel[i], 0.0, std)) for i in idx]


C4_SEED = 4
C5_GRAD_SEED = 5100


def c4_numel() -> List[int]:
    return sizes.c4_sizes()


def c5_numel() -> List[int]:
    return sizes.c5_sizes()

