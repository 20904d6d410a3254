"""Random and exhaustive op DAGs over every elementwise opcode, for the
fused-equals-unfused and fused-equals-oracle checks.

Every value carries an interval its elements lie in, from the inputs'
[-1.5, 1.5] (a u8 mask in {0, 1}); an op is drawn only where its domain
holds over that interval (sqrt of a nonnegative value, a divisor or a
reciprocal's operand away from zero) and its result stays within 1e6, so
no run hits an infinity or a NaN the two sides could reach differently."""
from __future__ import annotations

import itertools
import math

import numpy as np

from workloads.graph import Graph, TensorDesc

UNARY = ("exp", "tanh", "sigmoid", "relu", "gelu", "square", "sqrt", "recip", "neg")
IMM = (("add_imm", 0.5), ("mul_imm", -1.25))
BINARY = ("add", "sub", "mul", "div", "max", "min")
DMUL_SCALE = float(np.float32(1.0 / 0.9))
LIMIT = 1e6
GAP = 1e-2


def _gelu(x):
    return 0.5 * x * math.erfc(-x / math.sqrt(2.0))


def _sigmoid(x):
    # no exp of a large positive argument (an overflow in math.exp)
    return 1 / (1 + math.exp(-x)) if x >= 0 else math.exp(x) / (1 + math.exp(x))


def result_range(op, ranges, imm=0.0):
    """(lo, hi) of the op's result over its operands' intervals, or None
    when the op is not safe there."""
    if op in UNARY:
        lo, hi = ranges[0]
        if op == "exp":
            r = (math.exp(lo), math.exp(hi)) if hi <= 12 else None
        elif op == "tanh":
            r = (math.tanh(lo), math.tanh(hi))
        elif op == "sigmoid":
            r = (_sigmoid(lo), _sigmoid(hi))
        elif op == "relu":
            r = (max(lo, 0.0), max(hi, 0.0))
        elif op == "gelu":
            r = (min(-0.17, _gelu(lo)), max(_gelu(hi), 0.0))
        elif op == "square":
            m = max(lo * lo, hi * hi)
            r = (0.0 if lo <= 0 <= hi else min(lo * lo, hi * hi), m)
        elif op == "sqrt":
            r = (math.sqrt(lo), math.sqrt(hi)) if lo >= 0 else None
        elif op == "recip":
            r = (1 / hi, 1 / lo) if lo >= GAP or hi <= -GAP else None
        else:
            r = (-hi, -lo)
    elif op in ("add_imm", "mul_imm"):
        lo, hi = ranges[0]
        ends = (lo + imm, hi + imm) if op == "add_imm" else (lo * imm, hi * imm)
        r = (min(ends), max(ends))
    elif op == "dmul":
        (lo, hi) = ranges[0]
        r = (min(0.0, lo * DMUL_SCALE), max(0.0, hi * DMUL_SCALE))
    elif op == "add3":
        r = (sum(x[0] for x in ranges), sum(x[1] for x in ranges))
    else:
        (a0, a1), (b0, b1) = ranges
        if op == "add":
            r = (a0 + b0, a1 + b1)
        elif op == "sub":
            r = (a0 - b1, a1 - b0)
        elif op == "max":
            r = (max(a0, b0), max(a1, b1))
        elif op == "min":
            r = (min(a0, b0), min(a1, b1))
        elif op == "mul":
            p = (a0 * b0, a0 * b1, a1 * b0, a1 * b1)
            r = (min(p), max(p))
        else:  # div
            if not (b0 >= GAP or b1 <= -GAP):
                return None
            p = (a0 / b0, a0 / b1, a1 / b0, a1 / b1)
            r = (min(p), max(p))
    if r is None or max(abs(r[0]), abs(r[1])) > LIMIT:
        return None
    return r


def op_choices(avail, ranges, mask):
    """Every (op, inputs, imm) applicable to the available values."""
    out = []
    for op in UNARY:
        for a in avail:
            out.append((op, (a,), 0.0))
    for op, imm in IMM:
        for a in avail:
            out.append((op, (a,), imm))
    for op in BINARY:
        for a, b in itertools.product(avail, avail):
            out.append((op, (a, b), 0.0))
    for ins in itertools.product(avail, avail, avail):
        out.append(("add3", ins, 0.0))
    for a in avail:
        out.append(("dmul", (a, mask), DMUL_SCALE))
    ok = []
    for op, ins, imm in out:
        rs = [ranges[t] for t in ins if not (op == "dmul" and t == mask)]
        if result_range(op, rs, imm) is not None:
            ok.append((op, ins, imm))
    return ok


def _base(shape):
    g = Graph()
    x0, x1 = g.input("x0", "f32", shape), g.input("x1", "f32", shape)
    m = g.input("m", "u8", shape)
    return g, [x0, x1], m, {x0: (-1.5, 1.5), x1: (-1.5, 1.5), m: (0.0, 1.0)}


def _add(g, ranges, op, ins, imm, name, shape):
    rs = [ranges[t] for t in ins if not (op == "dmul" and g.tensors[t].dtype == "u8")]
    t = g.op(op, list(ins), name, "f32", shape, imm=imm)
    ranges[t] = result_range(op, rs, imm)
    return t


def _mark_outputs(g, extra=()):
    readers = {t for o in g.ops for t in o.inputs}
    for o in g.ops:
        t = o.output
        if t not in readers or t in extra:
            d = g.tensors[t]
            g.tensors[t] = TensorDesc(d.name, d.dtype, d.shape, "out")


def exhaustive_small(shape=(3, 5)):
    """Every DAG of one or two ops over x0, x1 (and the mask m): each as a
    list of (op, input names, imm) plus which intermediate is also an
    output."""
    g, avail, m, ranges = _base(shape)
    names = {avail[0]: "x0", avail[1]: "x1", m: "m"}
    dags = []
    for c1 in op_choices(avail, ranges, m):
        dags.append(((c1,), False))
        r1 = dict(ranges)
        r1[-1] = result_range(c1[0], [ranges[t] for t in c1[1] if t != m], c1[2])
        for c2 in op_choices(avail + [-1], r1, m):
            if -1 in c2[1]:
                dags.append(((c1, c2), False))
                dags.append(((c1, c2), True))
    return dags


THREE_VOCAB = ("tanh", "mul_imm", "sub", "dmul")


def exhaustive_three(vocab=THREE_VOCAB, shape=(3, 5)):
    """Every connected DAG of three ops over x0, x1 (and the mask m) drawn
    from `vocab` -- by default one transcendental, one immediate op, a
    binary op that does not commute and the masked multiply, so every
    operand wiring and every register path of three ops occurs: the first
    op's value is read by the second or the third, and the third reads the
    second's.  Same format as exhaustive_small (-1, -2: the first and second
    op's values)."""
    g, avail, m, ranges = _base(shape)

    def choices(av, rg):
        return [c for c in op_choices(av, rg, m) if c[0] in vocab]

    def rng_of(c, rg):
        return result_range(c[0], [rg[t] for t in c[1] if t != m], c[2])

    dags = []
    for c1 in choices(avail, ranges):
        r1 = dict(ranges)
        r1[-1] = rng_of(c1, ranges)
        for c2 in choices(avail + [-1], r1):
            r2 = dict(r1)
            r2[-2] = rng_of(c2, r1)
            for c3 in choices(avail + [-1, -2], r2):
                if -2 in c3[1] and (-1 in c2[1] or -1 in c3[1]):
                    dags.append(((c1, c2, c3), False))
    return dags


def combine(dags, shape):
    """One graph holding each small DAG as its own component over shared
    inputs x0, x1, m; returns (graph, per DAG its output tensor ids)."""
    g, avail, m, ranges = _base(shape)
    outs = []
    for k, (ops, t0_out) in enumerate(dags):
        made = []
        for j, (op, ins, imm) in enumerate(ops):
            real = [made[-t - 1] if t < 0 else t for t in ins]
            made.append(_add(g, ranges, op, real, imm, f"d{k}_{j}", shape))
        outs.append(made)
    readers = {t for o in g.ops for t in o.inputs}
    finals = []
    for (ops, t0_out), made in zip(dags, outs):
        mine = [t for t in made if t not in readers or (t0_out and t == made[0])]
        for t in mine:
            d = g.tensors[t]
            g.tensors[t] = TensorDesc(d.name, d.dtype, d.shape, "out")
        finals.append(mine)
    return g, finals


def random_dags(seed, count, n_ops, shape=(3, 5)):
    """DAGs of exactly n_ops ops drawn from every opcode: at each step the
    opcode uniformly among those applicable, then its operands uniformly;
    some intermediates are outputs too."""
    rng = np.random.default_rng(seed)
    for _ in range(count):
        g, avail, m, ranges = _base(shape)
        # half the DAGs open with a positive value (exp or sigmoid of an
        # input), so that sqrt, recip and div have an operand in their domain
        lead = rng.random() < 0.5
        for i in range(n_ops):
            if i == 0 and lead:
                op = ("exp", "sigmoid")[int(rng.integers(2))]
                avail.append(_add(g, ranges, op, (avail[int(rng.integers(2))],), 0.0, "t0", shape))
                continue
            by_op = {}
            for c in op_choices(avail, ranges, m):
                by_op.setdefault(c[0], []).append(c)
            names = sorted(by_op)
            ch = by_op[names[int(rng.integers(len(names)))]]
            op, ins, imm = ch[int(rng.integers(len(ch)))]
            avail.append(_add(g, ranges, op, ins, imm, f"t{i}", shape))
        extra = {o.output for o in g.ops if rng.random() < 0.15}
        _mark_outputs(g, extra)
        yield g
