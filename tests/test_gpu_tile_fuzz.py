"""Seeded random prefill-sized shapes (33-400 tokens, ragged M, N and K
within each mode's row rules) under randomly drawn forced tile variants:
the tile family with and without split-K, its stream-K form, and the
ping-pong kernels with their split-K.  Every output is checked against the
oracle (int8 accumulators exactly); a variant that does not apply to a
shape is rejected by the library and skipped."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_close, decode_out, reference, run, upload

lg = pytest.importorskip("epilogue_scaled_gemm_amd")
from epilogue_scaled_gemm_amd.sweep import SK_CANDIDATES, TILE_CANDIDATES  # noqa: E402

pytestmark = pytest.mark.gpu

QUANTS = ["bf16", "fp16", "fp8_dynamic", "w8a8_int8", "block_fp8", "mxfp4"]
ACTS = ["none", "relu", "gelu_tanh", "silu"]
SPECS = TILE_CANDIDATES + SK_CANDIDATES


def draw(count=60, seed=4343):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        q = QUANTS[i % len(QUANTS)]
        M = int(rng.integers(33, 401))
        if q == "block_fp8":
            N, K = 128 * int(rng.integers(1, 5)), 128 * int(rng.integers(1, 10))
        elif q == "mxfp4":
            N, K = int(rng.integers(1, 90)) * 8, 256 * int(rng.integers(1, 5))
        else:
            step = 8 if q in ("bf16", "fp16") else 16
            N, K = int(rng.integers(1, 700)), step * int(rng.integers(1, 90))
        spec = SPECS[int(rng.integers(0, len(SPECS)))]
        out.append((q, ACTS[int(rng.integers(0, 4))], M, N, K, bool(rng.integers(0, 2)),
                    bool(rng.integers(0, 2)), spec, i))
    return out


CASES = draw()


@pytest.fixture(scope="module")
def handle():
    h = lg.Handle()
    yield h
    h.close()


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-{c[2]}x{c[3]}x{c[4]}-{c[8]}" for c in CASES])
def test_forced_tile_variant_random_shape(handle, case):
    q, act, M, N, K, bias, res, spec, i = case
    p = synth.make_custom(q, act, M, N, K, seed=9000 + i, bias=bias, residual=res)
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
