"""GPU parity of the staged-activation decode mode (xs=1: each wave copies
its steps' activation bytes into LDS with direct-to-LDS loads and the lanes
read their fragments from there).  The products and their order are those of
the same variant without staging, so the outputs must be identical bit for
bit; they are also checked against the oracle (the int8 accumulator
exactly).  Covers e4m3, int8, block e4m3 and MXFP4 weights, ragged K tails
(e4m3), one to sixteen tokens and a split-K case."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_close, decode_out, dev

lg = pytest.importorskip("epilogue_scaled_gemm_amd")
pytestmark = pytest.mark.gpu

FP8_SHAPES = [(8, 1, 12), (8, 2, 16), (8, 4, 12), (8, 4, 24), (12, 1, 16)]
MX_SHAPES = [(8, 1, 16), (8, 2, 12), (8, 1, 24), (12, 1, 16)]
CASES = [("fp8_dynamic", "none", 1, 1040, 4096, True, False),
         ("fp8_dynamic", "gelu_tanh", 3, 528, 272, True, True),
         ("fp8_dynamic", "silu", 16, 6144, 1024, True, False),
         ("mxfp4", "none", 1, 1040, 4096, True, False),
         ("mxfp4", "relu", 5, 528, 256, False, True),
         ("mxfp4", "silu", 16, 272, 512, True, False),
         ("w8a8_int8", "silu", 4, 2064, 4096, False, False),
         ("block_fp8", "none", 3, 512, 3072, False, True),
         ("bf16", "gelu_tanh", 1, 1040, 4096, True, False),
         ("bf16", "silu", 9, 528, 1032, False, True),
         ("fp16", "relu", 5, 272, 520, True, True)]
I8_SHAPES = [(4, 4, 16), (8, 2, 16), (8, 4, 24), (4, 2, 32), (8, 1, 24)]
BLOCK_SHAPES = [(12, 1, 16), (8, 1, 16), (16, 1, 16)]
BF16_SHAPES = [(8, 1, 24), (8, 1, 16), (8, 2, 12)]


@pytest.fixture(scope="module")
def handle():
    h = lg.Handle()
    yield h
    h.close()


def run(handle, p, spec):
    C = torch.empty((p.M, p.N), dtype=torch.int16, device="cuda")
    handle.set_force(spec)
    try:
        handle.run(dev(p.A), dev(p.B), C, quant=p.quant, act=p.act, sa=dev(p.sa), sb=dev(p.sb),
                   alpha=p.alpha, bias=dev(p.bias), residual=dev(p.residual))
    finally:
        handle.set_force(None)
    torch.cuda.synchronize()
    return C.cpu()


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-M{c[2]}-N{c[3]}-K{c[4]}" for c in CASES])
def test_staged_activations_match(handle, case):
    quant, act, M, N, K, b, r = case
    p = synth.make_custom(quant, act, M, N, K, seed=3 * M + N + K, bias=b, residual=r)
    ref, _ = oracle.linear(quant, act, p.A, p.B, sa=p.sa, sb=p.sb, bias=p.bias,
                           residual=p.residual, alpha=p.alpha)
    shapes = {"mxfp4": MX_SHAPES, "w8a8_int8": I8_SHAPES, "block_fp8": BLOCK_SHAPES,
              "bf16": BF16_SHAPES, "fp16": BF16_SHAPES}.get(quant, FP8_SHAPES)
    specs = [f"decode swap=1 split=1 reduce=twopass waves={w} unroll={u} rows={rows}"
             for w, u, rows in shapes]
    specs.append("decode swap=1 split=2 reduce=lastwg waves=8 unroll=1 rows=16")
    staged = 0
    for spec in specs:
        handle.set_force(spec + " xs=1")
        used = "xs=1" in handle.describe(quant, M, N, K)
        handle.set_force(None)
        staged += used
        print(f"[stage] {quant} {M}x{N}x{K} {spec} staged={used}", flush=True)
        C1 = run(handle, p, spec + " xs=1")
        C0 = run(handle, p, spec)
        assert torch.equal(C1, C0), f"staged vs direct differ [{spec}]"
        assert_close(decode_out(C1, quant), ref, f"staged {quant} {M}x{N}x{K} [{spec}]")
        if quant == "w8a8_int8":
            Craw = torch.empty((M, N), dtype=torch.int32, device="cuda")
            handle.set_force(spec + " xs=1")
            try:
                handle.run(dev(p.A), dev(p.B), Craw, quant=quant, act="raw_acc", sa=dev(p.sa),
                           sb=dev(p.sb))
            finally:
                handle.set_force(None)
            torch.cuda.synchronize()
            _, acc = oracle.linear(quant, "none", p.A, p.B, p.sa, p.sb)
            assert np.array_equal(Craw.cpu().numpy(), acc), f"int8 accumulator [{spec}]"
    assert staged >= len(specs) - 2, "the staged mode was not used"


# Two token tiles (17..32 tokens): the variants compiled with staging there.
TWO_TILE = [("fp8_dynamic", "none", 24, 1040, 4096, True, False,
             [(8, 1, 24), (8, 1, 32), (8, 4, 24), (16, 1, 24), (16, 1, 32), (16, 2, 24)]),
            ("w8a8_int8", "silu", 32, 528, 1024, False, False, [(4, 2, 32)]),
            ("mxfp4", "gelu_tanh", 20, 272, 512, True, True, [(4, 2, 32), (8, 1, 24)]),
            ("block_fp8", "none", 17, 256, 1024, False, True,
             [(8, 2, 32), (8, 1, 32), (12, 1, 16), (16, 1, 16), (4, 2, 32), (16, 2, 16),
              (12, 2, 16)]),
            ("bf16", "relu", 30, 272, 1032, True, True, [(8, 1, 24), (8, 1, 32), (16, 1, 24), (16, 2, 32)]),
            ("w8a8_int8", "none", 20, 528, 4096, True, False, [(16, 1, 32)]),
            ("fp16", "gelu_tanh", 27, 272, 1024, True, True, [(16, 1, 24)])]


@pytest.mark.parametrize("case", TWO_TILE, ids=[f"{c[0]}-M{c[2]}" for c in TWO_TILE])
def test_staged_two_token_tiles(handle, case):
    quant, act, M, N, K, b, r, shapes = case
    p = synth.make_custom(quant, act, M, N, K, seed=5 * M + N, bias=b, residual=r)
    ref, acc = oracle.linear(quant, act, p.A, p.B, sa=p.sa, sb=p.sb, bias=p.bias,
                             residual=p.residual, alpha=p.alpha)
    for w, u, rows in shapes:
        spec = f"decode swap=1 split=1 reduce=twopass waves={w} unroll={u} rows={rows}"
        handle.set_force(spec + " xs=1")
        used = "xs=1" in handle.describe(quant, M, N, K)
        handle.set_force(None)
        print(f"[stage] {quant} {M}x{N}x{K} {spec} staged={used}", flush=True)
        assert used, f"staged mode not available for {spec}"
        C1 = run(handle, p, spec + " xs=1")
        try:
            C0 = run(handle, p, spec)
        except lg.LinGemmError:
            # No unstaged build of this shape: one-step batches run the same
            # products in the same order.
            C0 = run(handle, p, spec.replace(f"unroll={u}", "unroll=1") + " xs=1")
        assert torch.equal(C1, C0), f"staged vs direct differ [{spec}]"
        assert_close(decode_out(C1, quant), ref, f"staged {quant} {M}x{N}x{K} [{spec}]")


# Staged activations with K split across workgroups (17..32 tokens): the
# products and their order are those of the unstaged variant with the same
# split and reduction, so the outputs must be identical bit for bit (except
# under the atomic reduction, whose order of arrival is not fixed).  Block
# e4m3 at the workload's own size (N = 4096, K = 12288) and a small ragged
# one; fp8 per-channel and bf16 with a K tail.
SPLIT = [("block_fp8", "none", 32, 4096, 12288, False, True),
         ("block_fp8", "silu", 19, 384, 3072, True, False),
         ("fp8_dynamic", "gelu_tanh", 25, 528, 4112, True, True),
         ("bf16", "none", 17, 272, 8200, True, False)]
SPLIT_SPECS = [f"decode swap=1 split={sp} reduce={red} waves=8 unroll=1 rows=64"
               for sp in (2, 4) for red in ("twopass", "lastwg", "atomic")] + \
              ["decode swap=1 split=2 reduce=twopass waves=16 unroll=1 rows=32",
               "decode swap=1 split=4 reduce=twopass waves=8 unroll=1 rows=32"]


@pytest.mark.parametrize("case", SPLIT, ids=[f"{c[0]}-M{c[2]}-N{c[3]}-K{c[4]}" for c in SPLIT])
def test_staged_split_k_two_token_tiles(handle, case):
    quant, act, M, N, K, b, r = case
    p = synth.make_custom(quant, act, M, N, K, seed=13 * M + N, bias=b, residual=r)
    ref, _ = oracle.linear(quant, act, p.A, p.B, sa=p.sa, sb=p.sb, bias=p.bias,
                           residual=p.residual, alpha=p.alpha)
    staged = 0
    for spec in SPLIT_SPECS:
        handle.set_force(spec + " xs=1")
        used = "xs=1" in handle.describe(quant, M, N, K)
        handle.set_force(None)
        staged += used
        print(f"[stage-split] {quant} {M}x{N}x{K} {spec} staged={used}", flush=True)
        C1 = run(handle, p, spec + " xs=1")
        if "atomic" not in spec:
            C0 = run(handle, p, spec)
            assert torch.equal(C1, C0), f"staged vs direct differ [{spec}]"
        assert_close(decode_out(C1, quant), ref, f"staged {quant} {M}x{N}x{K} [{spec}]")
    assert staged >= 2, "the staged mode was not used"


# Widened e4m3 activations (xs=2): each wave widens its K range's
# activations once into LDS; the fragments, products and their order are
# those of the same variant without it, so the outputs must be identical bit
# for bit.  Ragged K (a 16-byte tail step), ragged N (masked weight rows),
# one to sixteen tokens, and split-K slices.
WIDE = [("fp8_dynamic", "none", 1, 1040, 4096, True, False),
        ("fp8_dynamic", "gelu_tanh", 3, 528, 272, True, True),
        ("fp8_dynamic", "silu", 8, 6144, 4096, True, False),
        ("fp8_dynamic", "relu", 16, 272, 1024, False, True),
        ("fp8_dynamic", "none", 5, 1040, 12304, True, False),
        ("block_fp8", "none", 3, 512, 3072, False, True),
        ("block_fp8", "silu", 9, 256, 1024, True, False)]
WIDE_SHAPES = [(8, 1, 12), (8, 2, 12), (8, 4, 12), (12, 1, 16), (16, 1, 16), (8, 1, 24),
               (4, 4, 16), (8, 2, 16), (16, 1, 24), (16, 2, 24)]


@pytest.mark.parametrize("case", WIDE, ids=[f"{c[0]}-M{c[2]}-N{c[3]}-K{c[4]}" for c in WIDE])
def test_widened_activations_match(handle, case):
    quant, act, M, N, K, b, r = case
    p = synth.make_custom(quant, act, M, N, K, seed=11 * M + N + K, bias=b, residual=r)
    ref, _ = oracle.linear(quant, act, p.A, p.B, sa=p.sa, sb=p.sb, bias=p.bias,
                           residual=p.residual, alpha=p.alpha)
    specs = [f"decode swap=1 split=1 reduce=twopass waves={w} unroll={u} rows={rows}"
             for w, u, rows in WIDE_SHAPES if quant != "block_fp8" or 128 % rows == 0]
    specs += ["decode swap=1 split=2 reduce=twopass waves=8 unroll=1 rows=16",
              "decode swap=1 split=4 reduce=lastwg waves=8 unroll=2 rows=16"]
    widened = 0
    for spec in specs:
        handle.set_force(spec + " xs=2")
        used = "xs=2" in handle.describe(quant, M, N, K)
        handle.set_force(None)
        widened += used
        print(f"[wide] {quant} {M}x{N}x{K} {spec} widened={used}", flush=True)
        C2 = run(handle, p, spec + " xs=2")
        C0 = run(handle, p, spec)
        assert torch.equal(C2, C0), f"widened vs direct differ [{spec}]"
        assert_close(decode_out(C2, quant), ref, f"widened {quant} {M}x{N}x{K} [{spec}]")
    assert widened >= 2, "the widened mode was not used"


def test_staged_only_shape_rejected_where_staging_does_not_apply(handle):
    # The two-step block e4m3 shapes exist only staged for two token tiles:
    # forcing one at a single-tile token count fails with an error, and
    # launches nothing.
    p = synth.make_custom("block_fp8", "none", 8, 256, 1024, seed=1, bias=False, residual=False)
    with pytest.raises(lg.LinGemmError, match="staged"):
        run(handle, p, "decode swap=1 split=1 reduce=twopass waves=16 unroll=2 rows=16 xs=1")
