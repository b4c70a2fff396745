"""Every measured entry of the built-in table beyond the decode range
(token counts 33 and up, written by the sweep) through the default dispatch:
the shape resolves to the entry's variant, and the output matches the oracle
at the ends of the entry's token range (sampled positions plus corners and
the last row / column; int8 accumulators bit-exact at those positions)."""
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_close, decode_out, reference, run, sample_positions

pytestmark = pytest.mark.gpu

lg = pytest.importorskip("epilogue_scaled_gemm_amd")

INC = os.path.join(os.path.dirname(lg.__file__), "csrc", "table_mi355x.inc")


def _entries():
    body = open(INC).read().split('R"TABLE(', 1)[1].split(')TABLE"', 1)[0]
    out = []
    for line in body.splitlines():
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        q, lo, hi, N, K, *spec = line.split()
        if int(lo) > 32:
            out.append((q, int(lo), int(hi), int(N), int(K), " ".join(spec)))
    return out


def _cfg(quant, N, K):
    for cfg, c in synth.WORKLOADS.items():
        if c["N"] == N and c["K"] == K and (c["quant"] == quant or
                                            (quant == "bf16" and c["quant"] == "bf16")):
            return cfg
    return None


ENTRIES = _entries()


@pytest.fixture(scope="module")
def handle():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    h = lg.Handle()
    yield h
    h.close()


@pytest.mark.parametrize("quant,lo,hi,N,K,spec", ENTRIES,
                         ids=[f"{q}-{N}x{K}-M{lo}-{hi}" for q, lo, hi, N, K, _ in ENTRIES])
def test_table_entry(handle, quant, lo, hi, N, K, spec):
    cfg = _cfg(quant, N, K)
    assert cfg is not None, f"no workload with {quant} {N}x{K}"
    for M in sorted({lo, hi}):
        p = synth.make(cfg, M)
        got = handle.describe(p.quant, p.M, p.N, p.K)
        print(f"[table] {quant} M={M} N={N} K={K} -> {got}", flush=True)
        assert got.split()[:5] == spec.split()[:5] or got.startswith(spec.split()[0]), (got, spec)
        for key in ("bm", "bn", "wm", "wn"):
            if f"{key}=" in spec:
                assert f"{key}={spec.split(key + '=')[1].split()[0]}" in got, (got, spec)
        im, inn = sample_positions(p.M, p.N, 3000, seed=M)
        if quant == "w8a8_int8":
            C = run(handle, p, raw=True)
            _, acc = oracle.linear_at(p.quant, "none", p.A, p.B, im, inn, sa=p.sa, sb=p.sb)
            assert np.array_equal(C.cpu().numpy()[im, inn], acc), f"M={M}: accumulators"
        C = run(handle, p)
        r, _ = reference(p, (im, inn))
        assert_close(decode_out(C, p.quant)[im, inn], r, f"{quant} M={M} [{got}]")
