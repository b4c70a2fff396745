"""Stream-K tile variants (sk = persistent workgroups per CU): the tiles' K
stages divided evenly among the workgroups, split tiles fixed up by a second
kernel that sums their pieces in order and applies the epilogue.  Through the
C ABI against the oracle: every stream-K tile shape, one and two workgroups
per CU, every quant mode, ragged M / N / K, a shape with a data-parallel
part (more than twice as many tiles as workgroups) and a shape with fewer K
stages than workgroups.  int8 accumulators bit-exact; the rest within the
pass rule."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_close, decode_out, reference, run, sample_positions, upload

pytestmark = pytest.mark.gpu

lg = pytest.importorskip("epilogue_scaled_gemm_amd")

SHAPES = [(128, 128, 2, 2), (64, 128, 1, 4), (128, 128, 2, 4), (256, 128, 2, 4), (256, 256, 2, 4)]
QUANTS = [("fp8_dynamic", "gelu_tanh"), ("w8a8_int8", "silu"), ("block_fp8", "none"),
          ("bf16", "silu"), ("mxfp4", "relu")]


@pytest.fixture(scope="module")
def handle():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    h = lg.Handle()
    yield h
    h.set_force(None)
    h.close()


def _run_forced(h, p, spec, raw=False):
    h.set_force(spec)
    try:
        got = h.describe(p.quant, p.M, p.N, p.K)
        print(f"[sk] {p.quant} {p.M}x{p.N}x{p.K} {spec} -> {got}", flush=True)
        assert "sk=" in got, got
        return run(h, p, upload(p), raw=raw)
    finally:
        h.set_force(None)


def _dims(quant, rt_ok):
    # block FP8 needs N, K in 128 blocks; MXFP4 K % 256
    if quant == "block_fp8":
        return [(96, 640, 1280), (300, 1152, 2048)]
    if quant == "mxfp4":
        return [(96, 640, 1280), (300, 1000, 2048)]
    return [(96, 650, 1296), (300, 1000, 2064)]


# 4-bit weight tiles need BN a multiple of 32 x waves (as in the plain form).
CASES = [(q, a, bm, bn, wm, wn) for q, a in QUANTS for bm, bn, wm, wn in SHAPES
         if q != "mxfp4" or bn % (32 * wm * wn) == 0]


@pytest.mark.parametrize("quant,act,bm,bn,wm,wn", CASES,
                         ids=[f"{q}-{a}x{b}w{c}x{d}" for q, _, a, b, c, d in CASES])
def test_stream_k_parity(handle, quant, act, bm, bn, wm, wn):
    for sk in (1, 2):
        for M, N, K in _dims(quant, True):
            p = synth.make_custom(quant, act, M, N, K, seed=M + N + sk, bias=True,
                                  residual=quant in ("block_fp8", "bf16"), alpha=0.5)
            spec = f"tile bm={bm} bn={bn} wm={wm} wn={wn} sk={sk}"
            if quant == "w8a8_int8":
                C = _run_forced(handle, p, spec, raw=True)
                _, acc = oracle.linear(p.quant, "none", p.A, p.B, p.sa, p.sb)
                assert np.array_equal(C.cpu().numpy(), acc), f"{spec} {M}x{N}x{K}: accumulators"
            C = _run_forced(handle, p, spec)
            r, _ = reference(p)
            assert_close(decode_out(C, p.quant), r, f"{spec} {M}x{N}x{K}")


def test_stream_k_data_parallel_part(handle):
    # 32 x 48 = 1536 tiles of 64 x 128 against 256 (or 512) workgroups: most
    # tiles go whole to their own workgroups, the last ones are split.
    p = synth.make_custom("fp8_dynamic", "silu", 2048, 6144, 1024, seed=4, bias=True)
    for sk in (1, 2):
        C = _run_forced(handle, p, f"tile bm=64 bn=128 wm=1 wn=4 sk={sk}")
        g = decode_out(C, p.quant)
        im, inn = sample_positions(p.M, p.N, 4000, seed=sk)
        # and every row of the last 64-row block (the stream-K tiles) in full
        cols = np.arange(0, p.N, 64) + 63 * (np.arange(0, p.N, 64) // 64 % 2)
        im = np.concatenate([im, np.repeat(np.arange(p.M - 64, p.M), cols.size)])
        inn = np.concatenate([inn, np.tile(cols, 64)])
        r, _ = reference(p, (im, inn))
        assert_close(g[im, inn], r, f"data-parallel + stream-K sk={sk}")


def test_stream_k_fewer_units_than_workgroups(handle):
    # One tile of two K stages: two workgroups, two pieces, one fix-up.
    p = synth.make_custom("w8a8_int8", "none", 33, 100, 256, seed=2, bias=False)
    C = _run_forced(handle, p, "tile bm=128 bn=128 wm=2 wn=2 sk=1", raw=True)
    _, acc = oracle.linear(p.quant, "none", p.A, p.B, p.sa, p.sb)
    assert np.array_equal(C.cpu().numpy(), acc)
    q = synth.make_custom("bf16", "gelu_tanh", 40, 64, 128, seed=3, bias=True)
    C = _run_forced(handle, q, "tile bm=64 bn=128 wm=1 wn=4 sk=2")
    r, _ = reference(q)
    assert_close(decode_out(C, q.quant), r, "one tile, one stage")


def test_stream_k_repeats_bitwise(handle):
    # Deterministic: the fix-up sums the pieces in a fixed order.
    p = synth.make_custom("fp8_dynamic", "none", 300, 1000, 2064, seed=9, bias=True)
    a = _run_forced(handle, p, "tile bm=128 bn=128 wm=2 wn=2 sk=1")
    b = _run_forced(handle, p, "tile bm=128 bn=128 wm=2 wn=2 sk=1")
    assert torch.equal(a, b)
