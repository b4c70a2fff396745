"""Seeded random decode-sized shapes (1-32 tokens, ragged N and K within
each mode's row rules) under randomly drawn forced decode variants: plain,
split-K (two-pass, last-arrival, atomic), staged and widened activations
(also staged with K split across workgroups),
one or two token tiles.  Every output is checked against the oracle (int8
accumulators exactly); a variant that does not apply to a shape is
rejected by the library and skipped."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_close, decode_out, reference, run, upload

lg = pytest.importorskip("epilogue_scaled_gemm_amd")
from epilogue_scaled_gemm_amd.sweep import (DECODE_CANDIDATES, WD_CANDIDATES,  # noqa: E402
                                            XS_CANDIDATES, XS_SPLIT_CANDIDATES)

pytestmark = pytest.mark.gpu

QUANTS = ["bf16", "fp16", "fp8_dynamic", "w8a8_int8", "block_fp8", "mxfp4"]
ACTS = ["none", "relu", "gelu_tanh", "silu"]
SPECS = DECODE_CANDIDATES + XS_CANDIDATES + WD_CANDIDATES


def draw(count=120, seed=4242, specs=SPECS, min_m=1):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        q = QUANTS[i % len(QUANTS)]
        M = int(rng.integers(min_m, 33))
        if q == "block_fp8":
            N, K = 128 * int(rng.integers(1, 5)), 128 * int(rng.integers(1, 10))
        elif q == "mxfp4":
            N, K = int(rng.integers(1, 90)) * 8, 256 * int(rng.integers(1, 5))
        else:
            step = 8 if q in ("bf16", "fp16") else 16
            N, K = int(rng.integers(1, 700)), step * int(rng.integers(1, 90))
        spec = specs[int(rng.integers(0, len(specs)))]
        out.append((q, ACTS[int(rng.integers(0, 4))], M, N, K, bool(rng.integers(0, 2)),
                    bool(rng.integers(0, 2)), spec, i))
    return out


CASES = draw()
# Staged activations with K split across workgroups (two-pass reduction),
# mostly at two token tiles, where those variants are used.
SPLIT_CASES = draw(36, seed=4545, specs=XS_SPLIT_CANDIDATES, min_m=9)


@pytest.fixture(scope="module")
def handle():
    h = lg.Handle()
    yield h
    h.close()


@pytest.mark.parametrize("case", CASES + SPLIT_CASES,
                         ids=[f"{c[0]}-{c[2]}x{c[3]}x{c[4]}-{c[8]}" for c in CASES] +
                             [f"split-{c[0]}-{c[2]}x{c[3]}x{c[4]}-{c[8]}" for c in SPLIT_CASES])
def test_forced_decode_variant_random_shape(handle, case):
    q, act, M, N, K, bias, res, spec, i = case
    if q == "block_fp8" and "rows=" in spec and 128 % int(spec.split("rows=")[1].split()[0]):
        pytest.skip("block FP8 needs rows dividing 128")
    p = synth.make_custom(q, act, M, N, K, seed=7000 + i, bias=bias, residual=res)
    print(f"[fuzz] {p.name} [{spec}]", flush=True)
    d = upload(p)
    handle.set_force(spec)
    try:
        try:
            out = run(handle, p, d)
        except lg.LinGemmError as ex:
            pytest.skip(f"variant does not apply: {ex}")
        r, _ = reference(p)
        assert_close(decode_out(out, q), r, f"{p.name} [{spec}]")
        if q == "w8a8_int8":
            _, acc = oracle.linear(q, "none", p.A, p.B, p.sa, p.sb)
            assert np.array_equal(run(handle, p, d, raw=True).cpu().numpy(), acc), spec
    finally:
        handle.set_force(None)
