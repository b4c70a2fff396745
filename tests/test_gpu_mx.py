"""GPU parity of the MXFP4-weight decode (bf16 activations, E2M1 weights with
an E8M0 scale per 32 K values) against the oracle: every compiled variant on
ragged shapes with each epilogue, the split-K reductions, and the full
6144 x 4096 workload at one and 32 tokens."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_close, decode_out, dev

lg = pytest.importorskip("epilogue_scaled_gemm_amd")
pytestmark = pytest.mark.gpu

# (waves, unroll, rows) compiled for MXFP4 weights
MX_SHAPES = [(8, 1, 16), (8, 2, 12), (16, 1, 16), (12, 1, 16), (8, 1, 32), (4, 2, 24),
             (8, 2, 32), (4, 1, 64), (8, 1, 48)]
CASES = [("none", 1, 1040, 4096, True, False), ("gelu_tanh", 5, 528, 256, True, True),
         ("silu", 17, 272, 512, False, False), ("relu", 32, 136, 1024, True, True)]


@pytest.fixture(scope="module")
def handle():
    h = lg.Handle()
    yield h
    h.close()


def make(act, M, N, K, b, r, seed):
    return synth.make_custom("mxfp4", act, M, N, K, seed=seed, bias=b, residual=r)


def run(handle, p, spec=None):
    C = torch.empty((p.M, p.N), dtype=torch.int16, device="cuda")
    handle.set_force(spec)
    try:
        handle.run(dev(p.A), dev(p.B), C, quant="mxfp4", act=p.act, sb=dev(p.sb), alpha=p.alpha,
                   bias=dev(p.bias), residual=dev(p.residual))
    finally:
        handle.set_force(None)
    torch.cuda.synchronize()
    return C


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-M{c[1]}-N{c[2]}-K{c[3]}" for c in CASES])
def test_mx_variants_match_oracle(handle, case):
    act, M, N, K, b, r = case
    p = make(act, M, N, K, b, r, seed=M + N + K)
    ref, _ = oracle.linear("mxfp4", act, p.A, p.B, sb=p.sb, bias=p.bias, residual=p.residual,
                           alpha=p.alpha)
    specs = [f"decode swap=1 split=1 reduce=twopass waves={w} unroll={u} rows={rows}"
             for w, u, rows in MX_SHAPES]
    specs += ["decode swap=1 split=2 reduce=twopass waves=8 unroll=1 rows=16",
              "decode swap=1 split=2 reduce=lastwg waves=8 unroll=2 rows=32",
              "decode swap=1 split=4 reduce=atomic waves=8 unroll=1 rows=16"]
    for spec in specs:
        print(f"[mx] {act} {M}x{N}x{K} {spec}", flush=True)
        C = run(handle, p, spec)
        assert_close(decode_out(C, "mxfp4"), ref, f"mxfp4 {M}x{N}x{K} [{spec}]")


@pytest.mark.parametrize("M", [1, 32])
def test_mx_full_workload(handle, M):
    p = synth.make(6, M)
    print(f"[mx] workload 6 M={M} -> {handle.describe('mxfp4', M, p.N, p.K)}", flush=True)
    ref, _ = oracle.linear("mxfp4", p.act, p.A, p.B, sb=p.sb, bias=p.bias)
    C = run(handle, p)
    assert_close(decode_out(C, "mxfp4"), ref, f"mxfp4 workload M={M}")


def test_mx_rejects_unsupported(handle):
    p = make("none", 4, 256, 512, False, False, seed=1)
    with pytest.raises(lg.LinGemmError):
        run(handle, p, "decode swap=1 split=1 reduce=twopass waves=4 unroll=4 rows=16")
    with pytest.raises(lg.LinGemmError):
        run(handle, p, "decode swap=0 split=1 reduce=twopass waves=8 unroll=2 rows=16")


# Tile shapes (bm, bn, wm, wn) compiled for 4-bit weights (bn a multiple of
# 32 x waves): prefill-sized token counts.
MX_TILES = [(256, 256, 2, 2), (128, 256, 2, 2), (256, 128, 2, 2), (128, 128, 2, 2),
            (64, 128, 1, 4), (256, 256, 2, 4)]
PF_CASES = [("gelu_tanh", 33, 272, 512, True, True), ("none", 100, 1040, 1024, True, False),
            ("silu", 300, 200, 256, False, True)]


@pytest.mark.parametrize("case", PF_CASES, ids=[f"{c[0]}-M{c[1]}-N{c[2]}-K{c[3]}" for c in PF_CASES])
def test_mx_tile_shapes_match_oracle(handle, case):
    act, M, N, K, b, r = case
    p = make(act, M, N, K, b, r, seed=M * 7 + N + K)
    ref, _ = oracle.linear("mxfp4", act, p.A, p.B, sb=p.sb, bias=p.bias, residual=p.residual,
                           alpha=p.alpha)
    for bm, bn, wm, wn in MX_TILES:
        spec = f"tile bm={bm} bn={bn} wm={wm} wn={wn} group=4"
        print(f"[mx] {act} {M}x{N}x{K} {spec}", flush=True)
        C = run(handle, p, spec)
        assert_close(decode_out(C, "mxfp4"), ref, f"mxfp4 {M}x{N}x{K} [{spec}]")
    for spec in ("tile bm=64 bn=128 wm=1 wn=4 group=4 split=4",
                 "tile bm=128 bn=128 wm=2 wn=2 group=4 split=2"):
        C = run(handle, p, spec)
        assert_close(decode_out(C, "mxfp4"), ref, f"mxfp4 {M}x{N}x{K} [{spec}]")
    C = run(handle, p)  # the table's choice
    assert_close(decode_out(C, "mxfp4"), ref, f"mxfp4 {M}x{N}x{K} [default]")


def test_mx_tile_rejects_uneven_weight_split(handle):
    p = make("none", 64, 256, 512, False, False, seed=2)
    with pytest.raises(lg.LinGemmError):
        run(handle, p, "tile bm=64 bn=64 wm=2 wn=2 group=4")


def test_mx_prefill_workload_sampled(handle):
    # The 6144 x 4096 MXFP4 weight at 4096 tokens, checked on sampled outputs
    # (every row and column band, plus the corners).
    p = synth.make(7, 4096)
    print(f"[mx] workload 7 M=4096 -> {handle.describe('mxfp4', 4096, p.N, p.K)}", flush=True)
    C = run(handle, p)
    got = decode_out(C, "mxfp4")
    rng = np.random.default_rng(4)
    im = np.concatenate([rng.integers(0, p.M, 3000), [0, 0, p.M - 1, p.M - 1]])
    inn = np.concatenate([rng.integers(0, p.N, 3000), [0, p.N - 1, 0, p.N - 1]])
    ref, _ = oracle.linear_at("mxfp4", p.act, p.A, p.B, im, inn, sb=p.sb, bias=p.bias)
    assert_close(got[im, inn], ref, "mxfp4 workload M=4096 (sampled)")
