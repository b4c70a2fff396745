"""Pins for the oracle's MXFP4-weight layer (bf16 activations, E2M1 weights,
one E8M0 scale per 32 consecutive K values; the format of the OCP
Microscaling v1.0 specification).

The E2M1 decode is checked against the specification's value table, the
E8M0 decode against torch's float8_e8m0fnu cast on every code, the layer
against an exact Fraction brute force on tiny shapes, and the packing (low
nibble = even k) and the scale-block indexing on one-hot inputs."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth

# The specification's table of E2M1 magnitudes for codes 0..7.
SPEC_E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_decode_matches_the_spec_table():
    for c in range(16):
        v = oracle.e2m1_to_f64(c)
        assert abs(v) == SPEC_E2M1[c & 7]
        assert (c >= 8) == (np.signbit(v))


def test_e8m0_decode_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).double().numpy()
    got = np.array([oracle.e8m0_to_f64(int(c)) for c in codes])
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert np.array_equal(got[:255], ref[:255])


def bf16_vals(codes):
    return torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).double().numpy()


def brute(A, Bp, S, bias=None):
    """Exact result with Fractions, decoding through the spec table and torch."""
    M, K = A.shape
    N = Bp.shape[0]
    a = bf16_vals(A)
    sc = torch.from_numpy(S).view(torch.float8_e8m0fnu).double().numpy()
    out = np.empty((M, N))
    for m in range(M):
        for n in range(N):
            s = Fraction(0)
            for k in range(K):
                code = (Bp[n, k // 2] >> (4 * (k & 1))) & 15
                w = Fraction(SPEC_E2M1[code & 7]) * (-1 if code & 8 else 1)
                s += Fraction(a[m, k]) * w * Fraction(sc[n, k // 32])
            if bias is not None:
                s += Fraction(bf16_vals(bias)[n])
            out[m, n] = float(s)
    return out


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tiny_shapes_exact(seed):
    rng = np.random.default_rng(seed)
    M, N, K = 2, 3, 96
    A = synth.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    Bp = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    S = rng.integers(110, 140, (N, K // 32), dtype=np.uint8)
    bias = synth.to_bf16_bits(rng.uniform(-0.5, 0.5, N).astype(np.float32))
    got, _ = oracle.linear("mxfp4", "none", A, Bp, sb=S, bias=bias)
    ref = brute(A, Bp, S, bias)
    assert np.allclose(got, ref, rtol=1e-15, atol=0)


def test_packing_and_scale_blocks_on_one_hot_inputs():
    K = 128
    Bp = np.zeros((4, K // 2), np.uint8)
    S = np.full((4, K // 32), 127, np.uint8)   # scale 1
    Bp[0, 0] = 0x20                           # k = 1 holds code 2 (1.0); k = 0 holds 0
    Bp[1, 0] = 0x02                           # k = 0 holds 1.0
    Bp[2, 20] = 0x07                          # k = 40 holds 6.0 ...
    S[2, 1] = 130                             # ... in block 1, scaled by 2^3
    Bp[3, 63] = 0xF0                          # k = 127 holds -6.0
    for k, want in ((1, [1.0, 0.0, 0.0, 0.0]), (0, [0.0, 1.0, 0.0, 0.0]),
                    (40, [0.0, 0.0, 48.0, 0.0]), (127, [0.0, 0.0, 0.0, -6.0])):
        a = np.zeros((1, K), np.float32)
        a[0, k] = 1.0
        got, _ = oracle.linear("mxfp4", "none", synth.to_bf16_bits(a), Bp, sb=S)
        assert list(got[0]) == want, k


def test_synth_quantiser_round_trip():
    rng = np.random.default_rng(4)
    w = (rng.standard_normal((8, 256)) * 0.02).astype(np.float32)
    Bp, S = synth.quant_mxfp4(w)
    eye = np.eye(256, dtype=np.float32)
    deq, _ = oracle.linear("mxfp4", "none", synth.to_bf16_bits(eye), Bp, sb=S)  # [256, 8]
    scale = np.ldexp(1.0, S.astype(np.int64) - 127).repeat(32, axis=1)           # [8, 256]
    v = np.abs(w) / scale
    # half the E2M1 step at |v|: 0.25 below 2, 0.5 below 4, 1 up to 6; the
    # shared exponent puts max|v| in [4, 8), and values above 6 saturate.
    half = np.where(v < 2, 0.25, np.where(v < 4, 0.5, 1.0)) * scale
    sat = v > 6
    assert np.all(np.abs(deq.T - w)[~sat] <= half[~sat] * (1 + 1e-6))
    assert np.all(np.abs(deq.T[sat]) == 6 * scale[sat])
