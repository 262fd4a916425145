"""Write the small worked examples under tests/golden/.

Every stored value comes from the exact-rational brute force in oracle/brute.py (and is
cross-checked against the C oracle before writing).  The inputs are chosen so that each
expected value can also be derived by hand; the derivation is written into the file.
Run:  python tests/golden/make_golden.py
"""
from __future__ import annotations

import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
from oracle import brute  # noqa: E402


def _fmt(a) -> str:
    return " ".join(str(v) for v in np.asarray(a).ravel().tolist())


def write(name: str, header: list[str], fields: dict[str, np.ndarray]):
    with open(os.path.join(HERE, name), "w") as f:
        for h in header:
            f.write(f"# {h}\n")
        for k, v in fields.items():
            v = np.asarray(v)
            f.write(f"{k} {v.dtype.str} {'x'.join(map(str, v.shape))}: {_fmt(v)}\n")


def quant_pow2():
    v = np.array([127, -64, 3, 0, 0.5, 1.5, 2.5, -2.5], np.float64)
    x = (v * 0.125).astype(np.float16)[None, :]
    q, s = brute.quant_act(x.view(np.uint16))
    qo, so = oracle.quant_act(x)
    assert np.array_equal(q, qo) and np.array_equal(s, so)
    write("quant_act_pow2_ties.txt", [
        "Per-token symmetric int8 activation quantisation (Quasar Sec. 3.2-3.3, online",
        "activation quantisation before the INT8 GEMM); reading: s = absmax/127, round half to even.",
        "x = 0.125 * [127, -64, 3, 0, 0.5, 1.5, 2.5, -2.5]: absmax = 15.875 so s = 0.125 exactly,",
        "x/s is exact and the half-integers are ties: 0.5 -> 0, 1.5 -> 2, 2.5 -> 2, -2.5 -> -2.",
    ], {"x_f16": x.astype(np.float32), "scale_f32": s, "x_q": q})


def w8a8_tiny():
    xq = np.array([[1, 2, 3], [-1, 0, 127]], np.int8)
    sx = np.array([0.5, 0.25], np.float32)
    w = np.array([[1, 1, 1], [2, -1, 0]], np.int8)
    sw = np.array([0.125, 2.0], np.float32)
    y, acc = brute.linear_w8a8(xq, sx, w, sw)
    yo, acco = oracle.linear_w8a8(xq, sx, w, sw)
    assert np.array_equal(acc, acco) and np.array_equal(y, yo.view(np.uint16))
    write("w8a8_tiny.txt", [
        "W8A8 linear (Quasar Sec. 3.3 'INT8 Gemm and Dequantization'): int32 dot products, then",
        "y = acc * s_x[m] * s_w[n].  acc = [[6, 0], [126, -2]];",
        "y = [[6*0.5*0.125, 0], [126*0.25*0.125, -2*0.25*2]] = [[0.375, 0], [3.9375, -1]] (all exact).",
    ], {"x_q": xq, "x_scale": sx, "w": w, "w_scale": sw, "acc": acc.astype(np.int32),
        "y_f16": y.view(np.float16).astype(np.float32)})


def w4a16_two_groups():
    K = 256
    codes = (np.arange(K) % 16).astype(np.uint32)[None, :]
    q = np.bitwise_or.reduce(codes.reshape(1, K // 8, 8) << (4 * np.arange(8, dtype=np.uint32)), axis=2).astype(np.uint32)
    s = np.array([[0.5, 0.25]], np.float16)
    z = np.array([[8, 0]], np.uint8)
    x = np.ones((1, K), np.float16)
    y = brute.linear_w4a16(x.view(np.uint16), q, s.view(np.uint16), z)
    yo = oracle.linear_w4a16(x, q, s, z)
    assert np.array_equal(y, yo.view(np.uint16))
    write("w4a16_two_groups.txt", [
        "W4A16 linear (Speculative Decoding Meets Quantization review: 4-bit weights, 16-bit",
        "activations in the verify forward); reading: group 128, w = (q - z) * s, nibble j of word i",
        "is k = 8i + j.  Codes q_k = k mod 16 (words 0x76543210, 0xFEDCBA98 alternating), x = 1:",
        "group 0: z = 8, s = 0.5: 8 * sum_{j<16} (j - 8) * 0.5 = 8 * (-8) * 0.5 = -32;",
        "group 1: z = 0, s = 0.25: 8 * 120 * 0.25 = 240;  y = 208.",
    ], {"x_f16": x.astype(np.float32), "qweight": q, "scales_f16": s.astype(np.float32), "zeros": z,
        "y_f16": y.view(np.float16).astype(np.float32)})


def verify_tiny():
    logits = np.array([
        [0.0, 2.0, 2.0, -1.0, 1.0],
        [3.0, -0.0, 3.0, 3.0, 0.0],
        [-2.0, -1.0, -1.0, -3.0, -1.0],
        [0.5, 0.25, 0.75, 0.75, 1.0],
    ], np.float16)
    a = brute.argmax(logits.view(np.uint16))
    draft = np.array([1, 0, 3], np.int32)
    n = brute.accept(draft, a)
    assert np.array_equal(a, oracle.argmax(logits)) and n == oracle.accept(draft, a)
    write("verify_tiny.txt", [
        "Greedy verify (Quasar Sec. 4.5: the top-1 prediction decides; Sec. 4.2 / Table 1: L =",
        "tokens per verify).  Row argmax with the lowest index on ties: [1, 0, 1, 4].  Draft",
        "[1, 0, 3]: positions 0 and 1 match, position 2 does not, so n_accept = 2 and the step",
        "emits draft[0..1] + argmax[2] (L = 3).",
    ], {"logits_f16": logits.astype(np.float32), "draft": draft, "argmax": a,
        "n_accept": np.array([n], np.int32)})


if __name__ == "__main__":
    quant_pow2()
    w8a8_tiny()
    w4a16_two_groups()
    verify_tiny()
    print("golden files written")
