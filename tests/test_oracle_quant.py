"""Pins for the oracle's dynamic activation quantization.

The rounding of a binary32 value to an E4M3FN code is checked against torch's
CPU cast (an independent implementation) on every finite code, every midpoint
between neighbouring codes and the binary32 values on either side of each
midpoint.  The int8 rounding is checked on exact halves (ties to even, a
closed form), and the grouping (rows, 1x128 blocks) on hand-built examples
whose scales are powers of two.  Random rows check the properties that hold
for any input: the group maximum maps to the format's maximum, and every
code is within half a step of x / s.
"""
import numpy as np
import pytest
import torch

import oracle


def to_bf16_codes(v):
    t = torch.tensor(np.asarray(v, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def e4m3_torch(v):
    """torch's CPU float32 -> float8_e4m3fn cast (round to nearest even)."""
    t = torch.tensor(np.asarray(v, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def e4m3_values():
    """Values of the positive finite E4M3FN codes 0x00 .. 0x7E (torch decode)."""
    codes = np.arange(127, dtype=np.uint8)
    return torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()


def probe_values():
    """Every code value, each midpoint and the binary32 neighbours of each
    midpoint, with both signs (all within [-448, 448])."""
    v = e4m3_values().astype(np.float32)
    mid = ((v[:-1].astype(np.float64) + v[1:]) / 2).astype(np.float32)  # exact
    up = np.nextafter(mid, np.float32(np.inf))
    dn = np.nextafter(mid, np.float32(-np.inf))
    pos = np.concatenate([v, mid, up, dn])
    return np.concatenate([pos, -pos])


def test_e4m3_rounding_matches_torch_on_codes_and_midpoints():
    vals = probe_values()
    got = np.array([oracle.f32_to_e4m3(float(x)) for x in vals], dtype=np.uint8)
    ref = e4m3_torch(vals)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(vals[i]), int(got[i]), int(ref[i])) for i in bad[:8]]


def test_e4m3_ties_go_to_even_and_saturate():
    # 1.0625 lies halfway between 1.0 (code 0x38) and 1.125 (0x39): even -> 0x38;
    # 1.1875 between 1.125 (0x39) and 1.25 (0x3A): even -> 0x3A.
    assert oracle.f32_to_e4m3(1.0625) == 0x38
    assert oracle.f32_to_e4m3(1.1875) == 0x3A
    # Beyond the largest finite value: saturate to +-448 (0x7E / 0xFE).
    assert oracle.f32_to_e4m3(448.0) == 0x7E
    assert oracle.f32_to_e4m3(470.0) == 0x7E
    assert oracle.f32_to_e4m3(1.0e6) == 0x7E
    assert oracle.f32_to_e4m3(-1.0e6) == 0xFE
    # Below half the smallest subnormal (2^-10): zero, sign kept.
    assert oracle.f32_to_e4m3(2.0 ** -11) == 0x00
    assert oracle.f32_to_e4m3(-(2.0 ** -11)) == 0x80
    assert oracle.f32_to_e4m3(-0.0) == 0x80


@pytest.mark.parametrize("x_dtype", ["bf16", "fp16"])
def test_unit_scale_row_gives_the_cast_codes(x_dtype):
    # A row whose maximum is 448 has scale 448 / 448 = 1, so its codes are the
    # plain casts of its values.  All code values and midpoints are exact in
    # bf16 and fp16 (four significant bits).
    v = e4m3_values().astype(np.float32)
    mid = ((v[:-1].astype(np.float64) + v[1:]) / 2).astype(np.float32)
    row = np.concatenate([v, mid, -v, -mid]).astype(np.float32)
    if x_dtype == "bf16":
        X = to_bf16_codes(row)[None, :]
    else:
        X = row.astype(np.float16).view(np.uint16)[None, :]
        assert np.array_equal(X.view(np.float16).astype(np.float32)[0], row)
    pad = (-X.shape[1]) % 16
    X = np.concatenate([X, np.zeros((1, pad), np.uint16)], axis=1)
    Q, s = oracle.dynamic_quant("fp8_token", X, x_dtype)
    assert s[0] == np.float32(1.0)
    assert np.array_equal(Q[0, :row.size], e4m3_torch(row))


def test_int8_rounds_halves_to_even():
    row = np.array([127, 2.5, 3.5, -2.5, -3.5, 0.5, -0.5, 126.5, 1.5, -1.5, 0, 100.25,
                    -100.75, 64, -127, 0.25], dtype=np.float32)
    expect = np.array([127, 2, 4, -2, -4, 0, 0, 126, 2, -2, 0, 100, -101, 64, -127, 0])
    Q, s = oracle.dynamic_quant("int8_token", to_bf16_codes(row)[None, :])
    assert s[0] == np.float32(1.0)
    assert np.array_equal(Q[0].astype(np.int64), expect)


def test_block_scales_are_per_128_wide_block():
    # Block 0 has maximum 448 (scale 1); block 1 maximum 7 (scale 7 / 448 =
    # 2^-6, so its codes are the casts of 64 x); block 2 is all zero (scale 1,
    # codes 0); block 3 has maximum 0.4375 (scale 2^-10).
    rng = np.random.default_rng(3)
    blocks = []
    for amax in (448.0, 7.0, 0.0, 0.4375):
        b = (rng.uniform(-1, 1, 128) * amax + 0.0).astype(np.float32)  # no -0.0
        b = torch.tensor(b).to(torch.bfloat16).float().numpy()
        if amax:
            b[rng.integers(128)] = amax * rng.choice([-1, 1])
        blocks.append(b)
    row = np.concatenate(blocks)
    Q, s = oracle.dynamic_quant("fp8_block", to_bf16_codes(row)[None, :])
    assert s.shape == (1, 4)
    assert list(s[0]) == [1.0, 2.0 ** -6, 1.0, 2.0 ** -10]
    assert np.array_equal(Q[0, 0:128], e4m3_torch(blocks[0]))
    assert np.array_equal(Q[0, 128:256], e4m3_torch(blocks[1] * 64))
    assert np.all(Q[0, 256:384] == 0)
    assert np.array_equal(Q[0, 384:512], e4m3_torch(blocks[3] * 1024))
    # And the token kind over the same row uses one scale for all of it.
    Qt, st = oracle.dynamic_quant("fp8_token", to_bf16_codes(row)[None, :])
    assert st[0] == np.float32(1.0)
    assert np.array_equal(Qt[0], e4m3_torch(row))


def test_zero_row_scale_one_codes_zero():
    X = np.zeros((2, 256), np.uint16)
    X[1, 5] = 0x8000  # -0.0
    for kind in ("fp8_token", "int8_token", "fp8_block"):
        Q, s = oracle.dynamic_quant(kind, X)
        assert np.all(s == 1.0)
        assert np.all(Q.view(np.uint8)[0] == 0)
    Q, _ = oracle.dynamic_quant("fp8_token", X)
    assert Q[1, 5] == 0x80  # the sign of -0 is kept


@pytest.mark.parametrize("kind", ["fp8_token", "int8_token", "fp8_block"])
def test_random_rows_max_maps_to_format_max_and_half_step_bound(kind):
    rng = np.random.default_rng(11)
    M, K = 24, 384
    x = (rng.standard_normal((M, K)) * rng.uniform(0.01, 30, (M, 1))).astype(np.float32)
    X = to_bf16_codes(x)
    xv = torch.from_numpy(X.view(np.int16)).view(torch.bfloat16).double().numpy()
    Q, s = oracle.dynamic_quant(kind, X)
    glen = 128 if kind == "fp8_block" else K
    xg = xv.reshape(M, K // glen, glen)
    sg = np.asarray(s, np.float64).reshape(M, K // glen, 1)
    if kind == "int8_token":
        qv = Q.astype(np.float64).reshape(xg.shape)
        qmax = 127.0
        assert np.all(np.abs(qv - xg / sg) <= 0.5 + 1e-5)
    else:
        qv = torch.from_numpy(Q.view(np.uint8)).view(torch.float8_e4m3fn).double().numpy()
        qv = qv.reshape(xg.shape)
        qmax = 448.0
        v = np.abs(xg / sg)
        # half the spacing of E4M3FN at |v|: 2^(e-4) for normals (e = exponent
        # of |v|), 2^-10 in the subnormal range; plus binary32 slack.
        e = np.floor(np.log2(np.maximum(v, 2.0 ** -6)))
        half = np.where(v < 2.0 ** -6, 2.0 ** -10, 2.0 ** (e - 4))
        assert np.all(np.abs(np.abs(qv) - v) <= half * (1 + 1e-6) + 1e-12)
    # the group maximum maps to +-qmax, and the scale is amax / qmax
    amax = np.abs(xg).max(axis=2, keepdims=True)
    at = np.abs(xg) == amax
    assert np.all(np.abs(qv[at]) == qmax)
    assert np.allclose(sg, amax / qmax, rtol=1e-7, atol=0)
