"""Pins for the oracle's grouped (mixture-of-experts) layer: one expert is
the plain layer, empty segments produce nothing, and each segment equals the
plain layer of its rows with its expert's weight (checked through an
independent Fraction brute force on tiny shapes)."""
from fractions import Fraction

import numpy as np
import torch

import oracle
import synth


def test_one_expert_is_the_plain_layer():
    g = synth.make_grouped("fp8_dynamic", "silu", [5], 64, 128, seed=1)
    r, _ = oracle.grouped_linear("fp8_dynamic", "silu", g["A"], g["Bs"], g["offsets"],
                                 sa=g["sa"], sbs=g["sbs"], biases=g["biases"])
    p, _ = oracle.linear("fp8_dynamic", "silu", g["A"], g["Bs"][0], g["sa"], g["sbs"][0],
                         g["biases"][0])
    assert np.array_equal(r, p)


def test_segments_use_their_own_expert_exactly():
    sizes = [2, 0, 1, 3]
    g = synth.make_grouped("w8a8_int8", "none", sizes, 8, 32, seed=2, bias=False)
    r, acc = oracle.grouped_linear("w8a8_int8", "none", g["A"], g["Bs"], g["offsets"],
                                   sa=g["sa"], sbs=g["sbs"])
    off = g["offsets"]
    for e in range(len(sizes)):
        for m in range(off[e], off[e + 1]):
            for n in range(8):
                s = sum(int(g["A"][m, k]) * int(g["Bs"][e][n, k]) for k in range(32))
                assert acc[m, n] == s
                want = Fraction(s) * Fraction(float(g["sa"][m])) * Fraction(float(g["sbs"][e][n]))
                assert abs(r[m, n] - float(want)) <= 1e-12 * max(1.0, abs(float(want)))


def test_empty_problem():
    g = synth.make_grouped("bf16", "none", [0, 0], 16, 64, seed=3)
    r, _ = oracle.grouped_linear("bf16", "none", g["A"], g["Bs"], g["offsets"],
                                 biases=g["biases"])
    assert r.shape == (0, 16)
