"""Pins for the oracle's element decoders and bf16 rounding.

The oracle decodes codes with its own closed forms; here they are checked
against library casts (torch / numpy CPU) and the format facts, exhaustively.
"""
import math
import struct

import numpy as np
import pytest
import torch

import oracle


def test_e4m3_all_codes_match_torch_cast():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    ours = np.array([oracle.e4m3_to_f64(int(c)) for c in codes])
    nan_ref = np.isnan(ref)
    assert np.array_equal(nan_ref, np.isnan(ours))
    assert np.array_equal(ref[~nan_ref].astype(np.float64), ours[~nan_ref])


def test_e4m3_format_facts():
    vals = {c: oracle.e4m3_to_f64(c) for c in range(256)}
    nan_codes = sorted(c for c, v in vals.items() if math.isnan(v))
    assert nan_codes == [0x7F, 0xFF]                 # no infinities, two NaNs
    finite = [v for v in vals.values() if not math.isnan(v)]
    assert len(finite) == 254
    assert max(finite) == 448.0 and min(finite) == -448.0
    assert min(v for v in finite if v > 0) == 2.0 ** -9 == 0.001953125
    assert all((v * 512.0).is_integer() for v in finite)   # multiples of 2^-9
    assert vals[0x38] == 1.0 and vals[0xB8] == -1.0 and vals[0x40] == 2.0


def test_bf16_decode_all_codes():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    ours = np.array([oracle.bf16_to_f64(int(b)) for b in bits[::7]])
    with np.errstate(invalid="ignore"):
        r = ref[::7].astype(np.float64)
    nan = np.isnan(r)
    assert np.array_equal(nan, np.isnan(ours))
    assert np.array_equal(r[~nan], ours[~nan])


def test_fp16_decode_all_codes():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    ours = np.array([oracle.fp16_to_f64(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    assert np.array_equal(ref[~nan], ours[~nan])


def _bf16_torch(x: float) -> int:
    t = torch.tensor([x], dtype=torch.float32).to(torch.bfloat16)
    return int(t.view(torch.int16).item()) & 0xFFFF


def test_bf16_rounding_matches_torch_on_fp32_values():
    rng = np.random.default_rng(7)
    raw = rng.integers(0, 2 ** 32, size=4000, dtype=np.uint64).astype(np.uint32)
    with np.errstate(invalid="ignore"):
        vals = raw.view(np.float32).astype(np.float64)
    # ties (exactly half way between bf16 neighbours), subnormals, overflow
    ties = [struct.unpack("<f", struct.pack("<I", (b << 16) | 0x8000))[0]
            for b in (0x3F80, 0x3F81, 0x0001, 0x0002, 0x7F7E, 0xBF80, 0xBF81)]
    specials = [0.0, -0.0, 1e-40, -1e-40, 3.4e38, -3.4e38, 3.3961775e38, 1.0, -2.5,
                float(np.float32(1.0 + 2 ** -8)), float(np.float32(1.0 + 3 * 2 ** -9))]
    specials = [float(np.float32(v)) for v in specials]  # fp32-representable inputs only
    for x in list(vals) + ties + specials:
        if math.isnan(x):
            assert oracle.f64_to_bf16(x) & 0x7FFF > 0x7F80
            continue
        assert oracle.f64_to_bf16(x) == _bf16_torch(x), x


def test_bf16_rounding_exact_on_fp64_inputs():
    # Values between bf16 neighbours that fp32 cannot hold: must round on the
    # exact value (1 + 2^-8 + 2^-40 lies just above the tie -> rounds up).
    assert oracle.f64_to_bf16(1.0 + 2 ** -8 + 2 ** -40) == 0x3F81
    assert oracle.f64_to_bf16(1.0 + 2 ** -8 - 2 ** -40) == 0x3F80
    assert oracle.f64_to_bf16(1.0 + 2 ** -8) == 0x3F80          # tie -> even
    assert oracle.f64_to_bf16(1e300) == 0x7F80
    assert oracle.f64_to_bf16(-1e300) == 0xFF80
