"""Pins for the oracle's layer computation, independent of the oracle itself.

Each test fixes a property the pages or the mathematics determine: exact
brute force with Fractions on tiny shapes (decoding through torch's casts,
not the oracle's), the GELU-tanh / SiLU closed forms, identity and permutation
weights (catch transposes and index slips), the block-scale closed form, the
transpose identity used by swap-AB, the K-split identity used by split-K, and
the printed sizes.  A dropped term, a wrong sign or index, or a transposed
operand in the oracle fails at least one of them.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_facts.json")
with open(GOLDEN) as f:
    FACTS = json.load(f)


# ------------------------------------------------------- independent decode
def dec_torch(quant, codes):
    codes = np.ascontiguousarray(codes)
    if quant in ("bf16",):
        return torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).float().double().numpy()
    if quant == "fp16":
        return codes.view(np.float16).astype(np.float64)
    if quant in ("fp8_dynamic", "block_fp8"):
        return torch.from_numpy(codes).view(torch.float8_e4m3fn).float().double().numpy()
    if quant == "w8a8_int8":
        return codes.astype(np.int64)
    raise ValueError(quant)


def dec16(quant, codes):
    return dec_torch("fp16" if quant == "fp16" else "bf16", codes)


def _torch_act(name):
    """The activations as torch's own fp64 CPU routines (an implementation
    independent of the oracle's C code)."""
    import torch.nn.functional as F

    def f(y):
        t = torch.tensor(float(y), dtype=torch.float64)
        if name == "gelu_tanh":
            return float(F.gelu(t, approximate="tanh"))
        if name == "silu":
            return float(F.silu(t))
        if name == "relu":
            return float(torch.relu(t))
        return float(y)
    return f


def gelu_erf(y):
    return float(torch.nn.functional.gelu(torch.tensor(float(y), dtype=torch.float64)))


ACTS = {name: _torch_act(name) for name in ("none", "relu", "gelu_tanh", "silu")}


def brute(p: synth.Problem):
    """Exact accumulators with Fractions, epilogue in Python floats."""
    A = dec_torch(p.quant, p.A)
    B = dec_torch(p.quant, p.B)
    bias = dec16(p.quant, p.bias) if p.bias is not None else None
    res = dec16(p.quant, p.residual) if p.residual is not None else None
    out = np.empty((p.M, p.N))
    accs = np.zeros((p.M, p.N), dtype=np.int64)
    for m in range(p.M):
        for n in range(p.N):
            if p.quant == "block_fp8":
                KB = p.K // 128
                y = Fraction(0)
                for kb in range(KB):
                    part = sum(Fraction(float(A[m, k])) * Fraction(float(B[n, k]))
                               for k in range(kb * 128, kb * 128 + 128))
                    y += Fraction(float(p.sa[m, kb])) * Fraction(float(p.sb[n // 128, kb])) * part
            else:
                acc = sum(Fraction(float(A[m, k])) * Fraction(float(B[n, k])) for k in range(p.K))
                if p.quant == "w8a8_int8":
                    accs[m, n] = int(acc)
                y = acc
                if p.quant in ("fp8_dynamic", "w8a8_int8"):
                    y = y * Fraction(float(p.sa[m])) * Fraction(float(p.sb[n]))
            if bias is not None:
                y += Fraction(float(bias[n]))
            v = ACTS[p.act](float(y)) * p.alpha
            if res is not None:
                v += float(res[m, n])
            out[m, n] = v
    return out, accs


BRUTE_CASES = [
    ("bf16", "gelu_tanh", 3, 5, 8, True, False, 1.0),
    ("fp16", "relu", 2, 7, 6, True, True, 0.5),
    ("fp8_dynamic", "none", 4, 3, 8, True, False, 1.0),
    ("fp8_dynamic", "silu", 1, 6, 5, False, True, 2.0),
    ("w8a8_int8", "silu", 3, 4, 7, False, False, 1.0),
    ("w8a8_int8", "gelu_tanh", 2, 5, 8, True, True, 0.5),
    ("block_fp8", "none", 2, 128, 256, False, True, 1.0),
]


@pytest.mark.parametrize("quant,act,M,N,K,bias,res,alpha", BRUTE_CASES)
def test_brute_force_fraction(quant, act, M, N, K, bias, res, alpha):
    p = synth.make_custom(quant, act, M, N, K, seed=11 + M * 7 + N, bias=bias, residual=res,
                          alpha=alpha, wstd=0.5)
    r, acc = oracle.linear(p.quant, p.act, **p.operands())
    b, bacc = brute(p)
    if quant == "w8a8_int8":
        assert np.array_equal(acc.astype(np.int64), bacc)
    np.testing.assert_allclose(r, b, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("quant", ["fp8_dynamic", "bf16"])
def test_fp_accumulator_is_exact(quant):
    # act none, unit scales, no bias: r is the raw sum, which fp64 holds
    # exactly for e4m3 (multiples of 2^-18) and bf16 products at this size.
    p = synth.make_custom(quant, "none", 3, 4, 64, seed=5, bias=False, wstd=1.0)
    if p.sa is not None:
        p.sa[:] = 1.0
        p.sb[:] = 1.0
    r, _ = oracle.linear(p.quant, "none", **p.operands())
    A, B = dec_torch(quant, p.A), dec_torch(quant, p.B)
    for m in range(3):
        for n in range(4):
            exact = sum(Fraction(float(A[m, k])) * Fraction(float(B[n, k])) for k in range(64))
            assert Fraction(r[m, n]) == exact


# ------------------------------------------------------ activation forms
# Source of the activation definitions: "Совместная работа Helion и
# TorchInductor: слияние операторов", section "Проектирование расширяемых
# эпилогов в Helion", the kernel listing's activation branches (code 1 ReLU,
# code 2 the tanh approximation of GELU with sqrt(2/pi) printed as 0.79788456
# and the cubic coefficient 0.044715).  SiLU is named in the section
# "Стратегии операторного слияния" without a formula: x * sigmoid(x).

ACT_GRID = np.concatenate([np.linspace(-10.0, 10.0, 20001),
                           [-40.0, -20.0, -12.5, 12.5, 20.0, 40.0, 1e-8, -1e-8, 3e-5, -3e-5]])


@pytest.mark.parametrize("name", ["gelu_tanh", "silu", "relu"])
def test_activation_matches_torch_fp64(name):
    # torch's CPU float64 gelu(approximate="tanh"), silu and relu are an
    # implementation of their own; the oracle must agree with them to the
    # last couple of ulps everywhere on a dense grid.  The absolute term
    # admits one or two ulps of difference between two libm tanh/exp
    # implementations where 1 + tanh(z) cancels (large negative x).
    import torch.nn.functional as F
    t = torch.from_numpy(ACT_GRID.copy())
    want = {"gelu_tanh": lambda: F.gelu(t, approximate="tanh"), "silu": lambda: F.silu(t),
            "relu": lambda: torch.relu(t)}[name]().numpy()
    got = np.array([oracle.act(name, float(x)) for x in ACT_GRID])
    bound = 1e-13 * np.abs(want) + 4e-16 * np.maximum(np.abs(ACT_GRID), 1.0)
    bad = np.abs(got - want) > bound
    assert not bad.any(), f"{name}: first mismatch at x={ACT_GRID[bad][0]!r}"


def test_gelu_constants_recovered_from_oracle_match_listing():
    # Read the two constants back out of the oracle's own outputs: for the
    # tanh form f(x) = x/2 * (1 + tanh(z)), z = c*x + c*kappa*x^3, so
    # z(x) = atanh(2 f(x)/x - 1) at two points fixes c and c*kappa.  c must be
    # the listing's 0.79788456 to its printed precision (and sqrt(2/pi)),
    # kappa must be the printed 0.044715.
    def z(x):
        return math.atanh(2.0 * oracle.act("gelu_tanh", x) / x - 1.0)
    x1, x2 = 0.5, 1.0
    c, ck = np.linalg.solve(np.array([[x1, x1 ** 3], [x2, x2 ** 3]]), [z(x1), z(x2)])
    printed_c = FACTS["gelu_tanh_sqrt_2_over_pi"]["value"]
    printed_kappa = FACTS["gelu_tanh_cubic_coefficient"]["value"]
    assert abs(c - printed_c) <= 5e-9          # 8 printed decimals
    assert abs(c - math.sqrt(2.0 / math.pi)) < 1e-13
    assert abs(ck / c - printed_kappa) < 1e-12
    # A third point checks that nothing beyond the cubic term is present.
    x3 = 1.7
    assert abs(z(x3) - (c * x3 + ck * x3 ** 3)) < 1e-13


@pytest.mark.parametrize("x", [-6.0, -2.5, -0.75, 0.3, 1.0, 4.0])
def test_silu_logit_is_identity(x):
    # SiLU is x * sigmoid(x): the logit of f(x)/x is x itself (a sigmoid of
    # any other slope, or a missing factor x, fails this).
    s = oracle.act("silu", x) / x
    assert math.log(s / (1.0 - s)) == pytest.approx(x, rel=1e-12, abs=1e-13)


@pytest.mark.parametrize("x", [0.1, 0.5, 1.0, 2.0, 3.0, 5.0])
def test_activation_odd_part_identity(x):
    # f(x) - f(-x) = x for GELU (either form) and SiLU.
    for name in ("gelu_tanh", "silu"):
        assert oracle.act(name, x) - oracle.act(name, -x) == pytest.approx(x, rel=1e-14)


def test_gelu_is_tanh_form_not_erf():
    # The tanh form differs from the erf form (torch's exact GELU) by more
    # than the parity tolerance near x = -3.4; an erf GELU in the oracle would
    # fail here.
    x = -3.44
    t, e = oracle.act("gelu_tanh", x), gelu_erf(x)
    assert abs(t - ACTS["gelu_tanh"](x)) < 1e-15
    assert abs(t - e) > 1e-2 * max(abs(e), 1e-3)
    # ... while the two forms stay within the approximation's known maximum
    # absolute gap (about 4.7e-4) everywhere.
    grid = np.linspace(-8, 8, 3201)
    gap = max(abs(oracle.act("gelu_tanh", float(v)) - gelu_erf(float(v))) for v in grid)
    assert 4.0e-4 < gap < 5.0e-4


def test_activation_fixed_points():
    assert oracle.act("gelu_tanh", 0.0) == 0.0 and oracle.act("silu", 0.0) == 0.0
    assert oracle.act("silu", 1.0) == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), rel=1e-15)
    assert oracle.act("gelu_tanh", 40.0) == 40.0          # tanh saturates
    assert abs(oracle.act("gelu_tanh", -40.0)) < 1e-300 or oracle.act("gelu_tanh", -40.0) == 0.0


# ------------------------------------------------------ structured weights
ONE = {"bf16": 0x3F80, "fp16": 0x3C00, "fp8_dynamic": 0x38, "w8a8_int8": 1}
CODE_T = {"bf16": np.uint16, "fp16": np.uint16, "fp8_dynamic": np.uint8, "w8a8_int8": np.int8}


@pytest.mark.parametrize("quant,act", [("bf16", "gelu_tanh"), ("fp16", "relu"),
                                       ("fp8_dynamic", "silu"), ("w8a8_int8", "silu")])
def test_identity_weight(quant, act):
    M, K = 5, 24
    p = synth.make_custom(quant, act, M, K, K, seed=3, bias=True, residual=True, alpha=0.75)
    B = np.zeros((K, K), dtype=CODE_T[quant])
    B[np.arange(K), np.arange(K)] = ONE[quant]
    sb = np.ones(K, dtype=np.float32) if p.sb is not None else None
    r, _ = oracle.linear(quant, act, p.A, B, p.sa, sb, p.bias, p.residual, 0.75)
    A = dec_torch(quant, p.A)
    bias, res = dec16(quant, p.bias), dec16(quant, p.residual)
    for m in range(M):
        s = float(p.sa[m]) if p.sa is not None else 1.0
        for n in range(K):
            want = ACTS[act](s * float(A[m, n]) + float(bias[n])) * 0.75 + float(res[m, n])
            assert r[m, n] == pytest.approx(want, rel=1e-14, abs=1e-14)


@pytest.mark.parametrize("quant", ["bf16", "fp8_dynamic", "w8a8_int8"])
def test_permutation_weight(quant):
    M, K = 4, 40
    p = synth.make_custom(quant, "none", M, K, K, seed=9, bias=False)
    perm = np.random.default_rng(1).permutation(K)
    B = np.zeros((K, K), dtype=CODE_T[quant])
    B[np.arange(K), perm] = ONE[quant]
    sa = np.ones(M, dtype=np.float32) if p.sa is not None else None
    sb = np.ones(K, dtype=np.float32) if p.sb is not None else None
    r, _ = oracle.linear(quant, "none", p.A, B, sa, sb)
    A = dec_torch(quant, p.A)
    assert np.array_equal(r, A[:, perm].astype(np.float64))


def test_block_scale_closed_form():
    M, N, K = 7, 384, 640
    KB, NB = K // 128, N // 128
    A = np.full((M, K), 0x38, dtype=np.uint8)
    B = np.full((N, K), 0x38, dtype=np.uint8)
    sa = np.array([[2.0 ** ((m + kb) % 5) for kb in range(KB)] for m in range(M)], np.float32)
    sb = np.array([[2.0 ** -((nb + 2 * kb) % 3) for kb in range(KB)] for nb in range(NB)],
                  np.float32)
    r, _ = oracle.linear("block_fp8", "none", A, B, sa, sb)
    for m in range(M):
        for n in range(N):
            want = 128 * sum(2.0 ** (((m + kb) % 5) - ((n // 128 + 2 * kb) % 3)) for kb in range(KB))
            assert r[m, n] == want


@pytest.mark.parametrize("quant", ["bf16", "fp16", "fp8_dynamic", "w8a8_int8"])
def test_transpose_identity(quant):
    # (A B^T)^T = B A^T: the identity swap-AB relies on.
    p = synth.make_custom(quant, "none", 6, 9, 48, seed=21, bias=False)
    r1, a1 = oracle.linear(quant, "none", p.A, p.B, p.sa, p.sb)
    r2, a2 = oracle.linear(quant, "none", p.B, p.A, p.sb, p.sa)
    np.testing.assert_allclose(r1.T, r2, rtol=1e-15, atol=0)
    if a1 is not None:
        assert np.array_equal(a1.T, a2)


@pytest.mark.parametrize("quant", ["fp8_dynamic", "w8a8_int8"])
def test_k_split_identity(quant):
    # Summing the raw accumulators of two K halves gives the full one (split-K).
    p = synth.make_custom(quant, "none", 3, 5, 256, seed=4, bias=False)
    ones_a = np.ones(3, np.float32)
    ones_b = np.ones(5, np.float32)
    full, af = oracle.linear(quant, "none", p.A, p.B, ones_a, ones_b)
    lo, al = oracle.linear(quant, "none", p.A[:, :128], p.B[:, :128], ones_a, ones_b)
    hi, ah = oracle.linear(quant, "none", p.A[:, 128:], p.B[:, 128:], ones_a, ones_b)
    assert np.array_equal(full, lo + hi)
    if af is not None:
        assert np.array_equal(af, al + ah)


def test_int8_overflow_is_reported():
    K = 140000  # > 131071: 127*127*K no longer fits int32
    A = np.full((1, K), 127, np.int8)
    B = np.full((1, K), 127, np.int8)
    with pytest.raises(ValueError):
        oracle.linear("w8a8_int8", "none", A, B, np.ones(1, np.float32), np.ones(1, np.float32))


def test_sampled_matches_full():
    p = synth.make_custom("fp8_dynamic", "silu", 9, 33, 256, seed=8, bias=True, residual=True,
                          alpha=0.5)
    r, _ = oracle.linear(p.quant, p.act, **p.operands())
    im = np.array([0, 8, 3, 5])
    inn = np.array([0, 32, 17, 1])
    s, _ = oracle.linear_at(p.quant, p.act, p.A, p.B, im, inn, sa=p.sa, sb=p.sb, bias=p.bias,
                            residual=p.residual, alpha=p.alpha)
    assert np.array_equal(s, r[im, inn])


def test_unfused_stages_compose_to_fused_definition():
    p = synth.make_custom("bf16", "gelu_tanh", 4, 6, 32, seed=2, bias=True, residual=True,
                          alpha=0.5)
    t, _ = oracle.linear("bf16", "none", p.A, p.B)
    t16 = np.array([[oracle.f64_to_bf16(v) for v in row] for row in t], np.uint16)
    u = oracle.unfused_stage2(t16, p.bias)
    u16 = np.array([[oracle.f64_to_bf16(v) for v in row] for row in u], np.uint16)
    o = oracle.unfused_stage3(u16, p.residual, 0.5)
    fused, _ = oracle.linear("bf16", "gelu_tanh", **p.operands())
    # Same definition up to the two intermediate bf16 roundings.
    assert np.all(np.abs(o - fused) <= 2 ** -6 * (np.abs(fused) + 1.0))


# --------------------------------------------------------- printed sizes
def test_printed_sizes():
    f = FACTS["fp16_4096x4096_intermediate_bytes"]
    assert 4096 * 4096 * 2 == f["bytes"] == 32 * 2 ** 20
    assert 4096 * 4096 == FACTS["unfused_buffer_elements"]["value"]
    # 6 vs 2 accesses per element: unfused writes T, U, out and reads
    # (A,B)->T, T, U; fused reads inputs once and writes once.
    acc = FACTS["vram_accesses_per_element"]["value"]
    assert acc["unfused_3_kernels"] == 3 * acc["fused_1_kernel"]


def test_synth_workload_shapes_follow_pages():
    assert list(synth.WORKLOADS[2]["Ms"]) == FACTS["num_tokens_tuned"]["value"]
    assert list(synth.WORKLOADS[3]["Ms"]) == FACTS["num_tokens_tuned"]["value"]
    p = synth.make(4, 1)
    assert p.sa.shape == (1, p.K // FACTS["scale_blocks"]["value"]["activation"][1])
    assert p.sb.shape == (p.N // 128, p.K // 128)
