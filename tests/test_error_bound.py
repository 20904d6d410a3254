"""Pins for the per-element comparator of tests/error_bound.py, on the CPU:
it asks bit-exactness where only IEEE ops lead to a value, exactly the
stated 1e-6 for a transcendental read straight out, and it catches planted
mistakes -- a transcendental off by a little more than the bar, an IEEE op
off by one ulp, a reduction off by more than its bar -- while passing an
evaluation whose transcendentals are off by a little less than the bar."""
import contextlib

import numpy as np
import pytest

from oracle import evaluate as oev
from oracle import ops as oops
from tests import dag_gen
from tests.error_bound import assert_within, run_with_bounds
from workloads import configs
from workloads.graph import Graph


def _inputs(g, seed):
    ins = {}
    for k, t in enumerate(g.inputs()):
        d = g.tensors[t]
        if d.dtype == "u8":
            ins[t] = (configs.tensor_values("f32", d.shape, "uniform", seed, k, 0.0, 1.0) >= 0.1).astype(np.uint8)
        else:
            ins[t] = configs.tensor_values("f32", d.shape, "uniform", seed, k, -1.5, 1.5)
    return ins


@contextlib.contextmanager
def planted(op, fn):
    """The oracle with one op replaced (a mistake planted on the CPU)."""
    old = oops.apply

    def apply(o, args, imm=0.0, shape=None):
        r = old(o, args, imm, shape)
        return fn(r, args) if o == op else r
    oops.apply = apply
    try:
        yield
    finally:
        oops.apply = old


def _fake_run(g, ins):
    groups = [[i] for i in range(len(g.ops))]
    return oev.evaluate(g, ins, stored=(), groups=groups)


def _check_all(g, ins, fake):
    vals, bound = run_with_bounds(g, ins, [[i] for i in range(len(g.ops))])
    for t in g.outputs():
        assert_within(fake[t], vals[t], bound[t], "f32", g.tensors[t].name)


def test_ieee_only_graphs_get_a_zero_bound():
    n = 0
    for g in dag_gen.random_dags(5, 800, 4):
        if any(o.op in ("exp", "tanh", "sigmoid", "gelu") for o in g.ops):
            continue
        _, bound = run_with_bounds(g, _inputs(g, 3), [[i] for i in range(len(g.ops))])
        for t in g.outputs():
            assert np.all(bound[t] == 0)
        n += 1
    assert n >= 40


def test_a_transcendental_read_straight_out_gets_the_bar():
    g = Graph()
    x = g.input("x", "f32", (4, 64))
    y = g.op("tanh", [x], "y", "f32", (4, 64), role="out")
    ins = _inputs(g, 7)
    vals, bound = run_with_bounds(g, ins, [[0]])
    w = np.abs(vals[y].astype(np.float64))
    assert np.allclose(bound[y], 1e-6 * w + 4 * 2.0 ** -149, rtol=0, atol=0)


@pytest.mark.parametrize("op", ["exp", "tanh", "sigmoid", "gelu"])
def test_transcendentals_a_little_inside_the_bar_pass_and_outside_fail(op):
    graphs = [g for g in dag_gen.random_dags(11, 400, 3) if any(o.op == op for o in g.ops)][:60]
    assert len(graphs) >= 10
    for g in graphs:
        ins = _inputs(g, 13)
        with planted(op, lambda r, a: (r.astype(np.float64) * (1 + 0.9e-6)).astype(np.float32)):
            fake = _fake_run(g, ins)
        _check_all(g, ins, fake)
    caught = 0
    for g in graphs:
        ins = _inputs(g, 13)
        with planted(op, lambda r, a: (r.astype(np.float64) * (1 + 3e-6)).astype(np.float32)):
            fake = _fake_run(g, ins)
        try:
            _check_all(g, ins, fake)
        except AssertionError:
            caught += 1
    assert caught >= len(graphs) // 2


@pytest.mark.parametrize("op", ["add", "mul", "div", "sqrt", "max", "dmul"])
def test_an_ieee_op_one_ulp_off_is_caught(op):
    """In graphs of IEEE ops only, where every value must be bit-exact, the
    op one ulp off is caught unless a later op hides it (a max or min of a
    larger value, a relu of a negative one)."""
    trans = ("exp", "tanh", "sigmoid", "gelu")
    graphs = [g for g in dag_gen.random_dags(17, 4000, 3)
              if any(o.op == op for o in g.ops) and not any(o.op in trans for o in g.ops)][:60]
    if op in ("div", "sqrt"):
        # a positive operand without a transcendental: x^2 + 1/2
        g = Graph()
        x0, x1 = g.input("x0", "f32", (3, 5)), g.input("x1", "f32", (3, 5))
        q = g.op("add_imm", [g.op("square", [x1], "q0", "f32", (3, 5))], "q", "f32", (3, 5), imm=0.5)
        if op == "div":
            g.op("div", [x0, q], "y", "f32", (3, 5), role="out")
        else:
            g.op("sqrt", [q], "y", "f32", (3, 5), role="out")
        graphs = [g]
    assert len(graphs) >= (1 if op in ("div", "sqrt") else 10)
    caught = 0
    for g in graphs:
        ins = _inputs(g, 19)
        with planted(op, lambda r, a: np.nextafter(r, np.float32(np.inf)).astype(np.float32)):
            fake = _fake_run(g, ins)
        try:
            _check_all(g, ins, fake)
        except AssertionError:
            caught += 1
    assert caught >= len(graphs) * 3 // 4


def test_a_row_sum_outside_its_bar_is_caught():
    g = Graph()
    x = g.input("x", "f32", (8, 512))
    e = g.op("exp", [x], "e", "f32", (8, 512))
    s = g.op("row_sum", [e], "s", "f32", (8, 1), role="out")
    ins = _inputs(g, 23)
    mag = np.exp(ins[x].astype(np.float64)).sum(axis=1, keepdims=True)
    with planted("row_sum", lambda r, a: (r + 0.5e-5 * mag).astype(np.float32)):
        ok = _fake_run(g, ins)
    _check_all(g, ins, ok)
    with planted("row_sum", lambda r, a: (r + 3e-5 * mag).astype(np.float32)):
        bad = _fake_run(g, ins)
    with pytest.raises(AssertionError):
        _check_all(g, ins, bad)


def test_sigmoid_and_add3_bounds_in_the_tails():
    """The derivative bound of sigmoid stays positive far in the tail (where
    sigmoid itself is tiny but not 0), and add3's bound counts the rounding
    of a + b as well as the result's."""
    from tests.error_bound import _sigmoid_d, _propagate, _ulp32
    z = np.array([0.0, 10.0, 40.0, 64.5, 100.0])
    assert np.allclose(_sigmoid_d(z), np.exp(-z) / (1 + np.exp(-z)) ** 2, rtol=1e-12, atol=0)
    assert (_sigmoid_d(z) > 0).all() and _sigmoid_d(64.5) == pytest.approx(np.exp(-64.5), rel=1e-12)
    # a graph whose add3 reads a value already off by a little
    g = Graph()
    x0 = g.input("x0", "f32", (1, 1))
    x1 = g.input("x1", "f32", (1, 1))
    t = g.op("exp", [x0], "t", "f32", (1, 1))
    g.op("add3", [x1, t, x0], "y", "f32", (1, 1), role="out")
    ins = {x0: np.full((1, 1), -4.0, np.float32), x1: np.full((1, 1), -0.34, np.float32)}
    vals, bound = run_with_bounds(g, ins, [[0], [1]])
    y = g.outputs()[0]
    a_plus_b = abs(-0.34) + float(np.exp(-4.0))
    assert bound[y][0, 0] >= float(_ulp32(vals[y])[0, 0] + _ulp32(np.array(a_plus_b))), bound[y]
