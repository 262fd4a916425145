"""Worked examples under tests/golden/ (hand-derivable, written by make_golden.py from the
exact-rational brute force) checked against the C oracle and against the closed forms
stated in each file."""
import os

import numpy as np

import oracle

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    out = {}
    with open(os.path.join(HERE, name)) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            head, vals = line.split(":", 1)
            key, dt, shape = head.split()
            shape = tuple(int(s) for s in shape.split("x"))
            out[key] = np.array([float(v) for v in vals.split()]).astype(np.dtype(dt)).reshape(shape)
    return out


def test_golden_quant_pow2_ties():
    g = load("quant_act_pow2_ties.txt")
    x = g["x_f16"].astype(np.float16)
    q, s = oracle.quant_act(x)
    np.testing.assert_array_equal(q, g["x_q"])
    np.testing.assert_array_equal(s, g["scale_f32"])
    np.testing.assert_array_equal(q[0], [127, -64, 3, 0, 0, 2, 2, -2])
    assert s[0] == 0.125


def test_golden_w8a8_tiny():
    g = load("w8a8_tiny.txt")
    y, acc = oracle.linear_w8a8(g["x_q"], g["x_scale"], g["w"], g["w_scale"])
    np.testing.assert_array_equal(acc, g["acc"])
    np.testing.assert_array_equal(y.astype(np.float32), g["y_f16"])
    np.testing.assert_array_equal(y.astype(np.float32), [[0.375, 0.0], [3.9375, -1.0]])


def test_golden_w4a16_two_groups():
    g = load("w4a16_two_groups.txt")
    assert g["qweight"][0, 0] == 0x76543210 and g["qweight"][0, 1] == 0xFEDCBA98
    y = oracle.linear_w4a16(g["x_f16"].astype(np.float16), g["qweight"], g["scales_f16"].astype(np.float16),
                            g["zeros"])
    np.testing.assert_array_equal(y.astype(np.float32), g["y_f16"])
    assert float(y[0, 0]) == 208.0


def test_golden_verify_tiny():
    g = load("verify_tiny.txt")
    a, n = oracle.verify_greedy(g["logits_f16"].astype(np.float16), g["draft"])
    np.testing.assert_array_equal(a, g["argmax"])
    np.testing.assert_array_equal(a, [1, 0, 1, 4])
    assert n == g["n_accept"][0] == 2
