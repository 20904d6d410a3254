"""Pins for the oracle's op table and its graph evaluation: closed forms,
identities between different ops, numerical integration, and special cases
that reduce to PyTorch / NumPy library routines."""
import math

import numpy as np
import pytest
import torch
from scipy import integrate

from oracle import evaluate as ev
from oracle import numerics, ops
from workloads import configs

F32 = np.float32


def ulp_diff_f32(a, b):
    ai = np.asarray(a, dtype=F32).view(np.int32).astype(np.int64)
    bi = np.asarray(b, dtype=F32).view(np.int32).astype(np.int64)
    ai = np.where(ai < 0, -(ai & 0x7FFFFFFF), ai)
    bi = np.where(bi < 0, -(bi & 0x7FFFFFFF), bi)
    return np.abs(ai - bi)


def test_closed_forms():
    assert ops.apply("sigmoid", [F32([0.0])])[0] == F32(0.5)
    assert ops.apply("gelu", [F32([0.0])])[0] == F32(0.0)
    assert ops.apply("exp", [F32([0.0])])[0] == F32(1.0)
    assert ops.apply("tanh", [F32([0.0])])[0] == F32(0.0)
    assert ops.apply("exp", [F32([math.log(2.0)])])[0] == pytest.approx(2.0, rel=1e-7)
    assert ops.apply("sqrt", [F32([4.0, 9.0, 0.25])]).tolist() == [2.0, 3.0, 0.5]
    assert ops.apply("recip", [F32([4.0, -0.5])]).tolist() == [0.25, -2.0]
    assert ops.apply("square", [F32([-3.0])])[0] == F32(9.0)
    assert ops.apply("neg", [F32([2.0])])[0] == F32(-2.0)
    assert ops.apply("add_imm", [F32([1.0])], 0.5)[0] == F32(1.5)
    assert ops.apply("mul_imm", [F32([3.0])], 0.5)[0] == F32(1.5)
    assert ops.apply("div", [F32([1.0]), F32([3.0])])[0] == F32(1.0) / F32(3.0)
    assert ops.apply("max", [F32([1.0]), F32([2.0])])[0] == 2.0
    assert ops.apply("min", [F32([1.0]), F32([2.0])])[0] == 1.0


def test_relu_gives_positive_zero():
    r = ops.apply("relu", [F32([-0.0, -1.0, 2.5, 0.0])])
    assert r.view(np.uint32).tolist() == [0, 0, F32(2.5).view(np.uint32), 0]


def test_gelu_is_x_times_the_normal_cdf():
    # Phi by numerical integration of the normal density: independent of erfc
    for z in [-6.0, -4.5, -3.0, -1.7, -0.3, 0.2, 0.9, 2.2, 5.0]:
        phi, _ = integrate.quad(lambda t: math.exp(-0.5 * t * t) / math.sqrt(2 * math.pi),
                                -np.inf, z, epsabs=0, epsrel=1e-13)
        want = F32(z * phi)
        got = ops.apply("gelu", [F32([z])])[0]
        assert ulp_diff_f32(got, want) <= 1, (z, got, want)


def test_gelu_matches_torch_exact_gelu_in_float64():
    x = np.linspace(-8, 8, 20001).astype(F32)
    want = torch.nn.functional.gelu(torch.from_numpy(x.astype(np.float64))).numpy().astype(F32)
    got = ops.apply("gelu", [x])
    # torch's float64 erf form loses relative accuracy deep in the negative
    # tail; compare where it is accurate and check the tail is tiny there
    ok = x > -5
    assert ulp_diff_f32(got[ok], want[ok]).max() <= 2
    assert np.all(np.abs(got[~ok]) < 1e-5)


def test_sigmoid_tanh_identities():
    z = np.linspace(-20, 20, 4001).astype(F32)
    s = ops.apply("sigmoid", [z]).astype(np.float64)
    s_neg = ops.apply("sigmoid", [-z]).astype(np.float64)
    assert np.max(np.abs(s + s_neg - 1.0)) < 2 ** -23
    # tanh(x) = 2 sigmoid(2x) - 1
    x = np.linspace(-5, 5, 2001).astype(F32)
    t = ops.apply("tanh", [x]).astype(np.float64)
    s2 = ops.apply("sigmoid", [(2 * x).astype(F32)]).astype(np.float64)
    assert np.max(np.abs(t - (2 * s2 - 1))) < 4e-7
    # exp(a) * exp(b) ~ exp(a + b)
    a = np.linspace(-3, 3, 101).astype(F32)
    e = ops.apply("exp", [a]).astype(np.float64)
    assert np.max(np.abs(e * e[::-1] - 1.0)) < 1e-6


def test_add3_is_left_to_right():
    a, b, c = F32([1e8]), F32([-1e8]), F32([1.0])
    assert ops.apply("add3", [a, b, c])[0] == F32(1.0)     # (a+b)+c
    assert (a + (b + c))[0] == F32(0.0)                       # the other order differs


def test_dmul_scales_then_masks():
    h = F32([3.0, -2.0, 5.0])
    m = F32([1.0, 1.0, 0.0])
    s = float(F32(1.0 / 0.9))
    r = ops.apply("dmul", [h, m], s)
    assert r[0] == F32(3.0) * F32(s) and r[1] == F32(-2.0) * F32(s) and r[2] == 0.0
    assert np.array_equal(ops.apply("dmul", [h, F32([1, 1, 1])], 1.0), h)


def test_row_reductions():
    ones = np.ones((3, 4096), dtype=F32)
    assert ops.apply("row_sum", [ones]).tolist() == [[4096.0]] * 3
    c = np.full((2, 1024), F32(0.3), dtype=F32)
    assert np.all(ops.apply("row_mean", [c]) == F32(0.3))
    ints = np.arange(12, dtype=F32).reshape(3, 4)
    assert ops.apply("row_sum", [ints]).ravel().tolist() == [6.0, 22.0, 38.0]
    assert ops.apply("row_mean", [ints]).ravel().tolist() == [1.5, 5.5, 9.5]


# --------------------------------------------------------------- graphs
def test_c1_matches_torch_float64_sigmoid():
    g = configs.c1_graph(16, 40)
    ins = configs.c1_inputs(g)
    _, out = ev.run(g, ins)
    x, a, b = (torch.from_numpy(ins[t]) for t in g.inputs())
    prod = (x * a) * b                                  # fp32 IEEE products
    want = torch.sigmoid(prod.double()).float().numpy()
    assert np.array_equal(out[g.outputs()[0]], want)


def test_c2_matches_torch_fp32_then_bf16():
    g = configs.c2_graph(12, 40)                         # non-square: catches axis mix-ups
    ins = configs.c2_inputs(g)
    _, out = ev.run(g, ins)
    X, bias, R = (torch.from_numpy(numerics.bf16_to_f32(ins[t])) for t in g.inputs())
    want = (torch.relu(X + bias) + R).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(out[g.outputs()[0]], want)


def test_c2_with_zero_bias_and_residual_is_relu():
    g = configs.c2_graph(8, 24)
    ins = configs.c2_inputs(g)
    X, bias, R = g.inputs()
    ins[bias] = np.zeros_like(ins[bias])
    ins[R] = np.zeros_like(ins[R])
    _, out = ev.run(g, ins)
    x = numerics.bf16_to_f32(ins[X])
    assert np.array_equal(out[g.outputs()[0]], numerics.f32_to_bf16(np.where(x > 0, x, F32(0))))


def test_c3_rows_of_zero_sum_to_width_and_match_float64():
    g = configs.c3_graph(4, 4096)
    ins = configs.c3_inputs(g)
    (P,) = g.inputs()
    zero = {P: np.zeros_like(ins[P])}
    _, out = ev.run(g, zero)
    assert out[g.outputs()[0]].ravel().tolist() == [4096.0] * 4
    _, out = ev.run(g, ins)
    p = numerics.bf16_to_f32(ins[P]).astype(np.float64)
    want = (np.exp(p) + 0.5 * p + np.tanh(p)).sum(axis=1)
    got = out[g.outputs()[0]].ravel().astype(np.float64)
    assert np.max(np.abs(got - want) / np.abs(want)) < 1e-6


def test_c3_head_op_variant_is_the_same_function():
    g0, g1 = configs.c3_graph(3, 64), configs.c3_graph(3, 64, head_op=True)
    ins = configs.c3_inputs(g0)
    _, o0 = ev.run(g0, ins)
    _, o1 = ev.run(g1, ins)
    assert np.array_equal(o0[g0.outputs()[0]], o1[g1.outputs()[0]])


def test_layernorm_matches_torch_float64():
    g = configs.layernorm_graph(16, 256)
    ins = configs.layernorm_inputs(g, 5000)
    _, out = ev.run(g, ins)
    X, gamma, beta = (torch.from_numpy(numerics.bf16_to_f32(ins[t])).double() for t in g.inputs())
    want = torch.nn.functional.layer_norm(X, (256,), gamma, beta, eps=configs.LN_EPS)
    got = numerics.bf16_to_f32(out[g.outputs()[0]]).astype(np.float64)
    err = np.abs(got - want.numpy())
    # one bf16 rounding of a value of size ~|y| (plus fp32 op noise)
    assert np.all(err <= 2 ** -8 * np.abs(want.numpy()) + 1e-5)


def test_layernorm_of_constant_rows_is_beta():
    g = configs.layernorm_graph(4, 64)
    ins = configs.layernorm_inputs(g, 5001)
    X, gamma, beta = g.inputs()
    ins[X] = np.full_like(ins[X], numerics.f32_to_bf16(F32([0.75]))[0])
    _, out = ev.run(g, ins)
    assert np.array_equal(out[g.outputs()[0]], np.broadcast_to(ins[beta], (4, 64)))


def test_layernorm_unit_affine_gives_zero_mean_and_var_ratio():
    g = configs.layernorm_graph(8, 1024)
    ins = configs.layernorm_inputs(g, 5002)
    X, gamma, beta = g.inputs()
    ins[gamma] = numerics.f32_to_bf16(np.ones(1024, dtype=F32))
    ins[beta] = np.zeros_like(ins[beta])
    vals, out = ev.run(g, ins)
    y = numerics.bf16_to_f32(out[g.outputs()[0]]).astype(np.float64)
    x = numerics.bf16_to_f32(ins[X]).astype(np.float64)
    v = x.var(axis=1)
    assert np.all(np.abs(y.mean(axis=1)) < 5e-3)
    assert np.allclose(y.var(axis=1), v / (v + configs.LN_EPS), rtol=1e-2)


def test_gelu_group_matches_torch():
    g = configs.gelu_graph(8, 96)
    ins = configs.gelu_inputs(g, 5000)
    _, out = ev.run(g, ins)
    A, b = (torch.from_numpy(numerics.bf16_to_f32(ins[t])) for t in g.inputs())
    z = (A + b).double()                                  # fp32 add, then exact widening
    want = torch.nn.functional.gelu(z).float()
    got = torch.from_numpy(numerics.bf16_to_f32(out[g.outputs()[0]]))
    wb = want.to(torch.bfloat16).float()
    assert torch.equal(got[z > -5], wb[z > -5])


def test_row_max_closed_cases_and_brute_force():
    x = F32([[1.0, 5.0, -2.0], [0.0, -3.0, -1.0], [-7.0, -7.5, -6.25]])
    assert ops.apply("row_max", [x]).ravel().tolist() == [5.0, 0.0, -6.25]
    # an empty row gives the identity of max
    e = ops.apply("row_max", [np.zeros((2, 0), dtype=F32)])
    assert e.shape == (2, 1) and np.all(np.isneginf(e))
    # a plain Python scan with ">" on small random rows
    rng = np.random.default_rng(11)
    for _ in range(50):
        r, c = int(rng.integers(1, 5)), int(rng.integers(1, 9))
        a = rng.normal(-1.0, 3.0, size=(r, c)).astype(F32)
        got = ops.apply("row_max", [a]).ravel()
        for i in range(r):
            best = a[i, 0]
            for v in a[i, 1:]:
                if v > best:
                    best = v
            assert got[i] == best


def test_softmax_group_matches_torch_softmax():
    """The softmax graph (max, exp(x - max), sum, times 1/sum) against
    torch's float64 softmax: the bf16 outputs are the float64 result
    rounded, or its bf16 neighbour."""
    g = configs.softmax_graph(8, 96)
    ins = configs.softmax_inputs(g, 5001)
    _, out = ev.run(g, ins)
    (X,) = g.inputs()
    x = torch.from_numpy(numerics.bf16_to_f32(ins[X]).astype(np.float64))
    want = torch.softmax(x, dim=1).float().to(torch.bfloat16).view(torch.int16).numpy().astype(np.int32)
    got = out[g.outputs()[0]].astype(np.int32)
    assert np.abs(got - want).max() <= 1
    # and the float64 rows of the rounded result sum to one within rounding
    y = numerics.bf16_to_f32(out[g.outputs()[0]]).astype(np.float64)
    assert np.all(np.abs(y.sum(axis=1) - 1.0) <= 96 * 2.0 ** -8 * y.max(axis=1))


def test_dropout_special_masks():
    g = configs.dropout_graph(4, 32)
    ins = configs.dropout_inputs(g, 5000)
    h, m, R = g.inputs()
    hf, Rf = numerics.bf16_to_f32(ins[h]), numerics.bf16_to_f32(ins[R])
    # mask of ones with scale one: h + R, one rounding
    g1 = configs.dropout_graph(4, 32, p=0.0)
    ins1 = dict(ins)
    ins1[m] = np.ones_like(ins[m])
    _, out = ev.run(g1, ins1)
    assert np.array_equal(out[g1.outputs()[0]], numerics.f32_to_bf16(hf + Rf))
    # mask of zeros: exactly R
    ins0 = dict(ins)
    ins0[m] = np.zeros_like(ins[m])
    _, out = ev.run(g, ins0)
    assert np.array_equal(out[g.outputs()[0]], ins[R])
    # torch, same op order
    _, out = ev.run(g, ins)
    s = torch.tensor(F32(1.0 / 0.9))
    want = ((torch.from_numpy(hf) * s) * torch.from_numpy(ins[m].astype(F32)) + torch.from_numpy(Rf))
    assert np.array_equal(out[g.outputs()[0]],
                          want.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))


def test_stored_intermediates_are_rounded_to_their_dtype():
    g = configs.c2_graph(4, 16)
    ins = configs.c2_inputs(g)
    X, bias, R = g.inputs()
    tmp = g.ops[0].output
    v_fused = ev.evaluate(g, ins)
    v_unf = ev.evaluate(g, ins, stored={tmp})
    assert np.array_equal(v_unf[tmp], numerics.round_to(v_fused[tmp], "bf16"))


def test_shape_errors_are_reported():
    from workloads.graph import Graph
    g = Graph()
    a = g.input("a", "f32", (4, 5))
    b = g.input("b", "f32", (5, 4))
    g.op("add", [a, b], "c", "f32", (4, 5), role="out")
    with pytest.raises(ValueError):
        ev.evaluate(g, {a: np.zeros((4, 5), F32), b: np.zeros((5, 4), F32)})
