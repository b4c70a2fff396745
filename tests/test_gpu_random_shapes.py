"""Seeded random shapes through the default dispatch (table, automatic
split-K factors, decode / tile / ping-pong families) in every quant mode,
against the oracle: int8 raw accumulators bit-exact, every other output
within the relative tolerance.  Shapes are drawn within each mode's
documented requirements (16-byte rows, 128-multiples for block FP8, K a
multiple of 256 for MXFP4) and span one token to a few hundred, with
ragged N and K tails."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_close, decode_out, reference, run, upload

lg = pytest.importorskip("epilogue_scaled_gemm_amd")
pytestmark = pytest.mark.gpu

QUANTS = ["bf16", "fp16", "fp8_dynamic", "w8a8_int8", "block_fp8", "mxfp4"]
ACTS = ["none", "relu", "gelu_tanh", "silu"]


def draw_shapes(count=48, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        q = QUANTS[i % len(QUANTS)]
        M = int(rng.choice([1, 2, 3, 7, 16, 17, 31, 32, 33, 64, 100, 257, 300]))
        if q == "block_fp8":
            N, K = 128 * int(rng.integers(1, 6)), 128 * int(rng.integers(1, 9))
        elif q == "mxfp4":
            N, K = int(rng.integers(1, 90)) * 8, 256 * int(rng.integers(1, 5))
        else:
            step = 8 if q in ("bf16", "fp16") else 16
            N, K = int(rng.integers(1, 700)), step * int(rng.integers(1, 80))
        out.append((q, ACTS[int(rng.integers(0, 4))], M, N, K, bool(rng.integers(0, 2)),
                    bool(rng.integers(0, 2)), float(rng.choice([1.0, 0.5, 2.0])), i))
    return out


SHAPES = draw_shapes()


@pytest.fixture(scope="module")
def handle():
    h = lg.Handle()
    yield h
    h.close()


@pytest.mark.parametrize("case", SHAPES, ids=[f"{c[0]}-{c[2]}x{c[3]}x{c[4]}" for c in SHAPES])
def test_random_shape_default_dispatch(handle, case):
    q, act, M, N, K, bias, res, alpha, seed = case
    p = synth.make_custom(q, act, M, N, K, seed=1000 + seed, bias=bias, residual=res, alpha=alpha)
    print(f"[random] {p.name} -> {handle.describe(q, M, N, K)}", flush=True)
    d = upload(p)
    r, _ = reference(p)
    assert_close(decode_out(run(handle, p, d), q), r, f"{p.name} [{handle.describe(q, M, N, K)}]")
    if q == "w8a8_int8":
        _, acc = oracle.linear(q, "none", p.A, p.B, p.sa, p.sb)
        assert np.array_equal(run(handle, p, d, raw=True).cpu().numpy(), acc)
