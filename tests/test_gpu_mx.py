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
