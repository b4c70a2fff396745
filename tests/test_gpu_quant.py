"""GPU parity of the dynamic activation quantization (lin_gemm_quantize) and
of the quantize-then-layer call (lin_gemm_run_dynamic) against the oracle.

Codes and scales are integer / binary32 decisions taken in the same precision
on both sides, so they must match bit for bit.  The layer output after
dynamic quantization follows the usual pass rule; the int8 accumulator is
exact.  Shapes span one and several 16-byte chunks per thread, rows longer
than the kernel's register cache (K > 8192), ragged block counts, one token
and many.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_close, decode_out, dev

lg = pytest.importorskip("epilogue_scaled_gemm_amd")
pytestmark = pytest.mark.gpu

KINDS = ["fp8_token", "int8_token", "fp8_block"]
SHAPES = [(1, 4096), (32, 4096), (7, 272), (3, 16), (33, 8320), (300, 1024), (2, 128),
          (5, 12288)]


@pytest.fixture(scope="module")
def handle():
    h = lg.Handle()
    yield h
    h.close()


def gpu_quantize(h, X, kind, x_dtype):
    M, K = X.shape
    Xd = dev(X)
    Q = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    S = torch.empty((M, K // 128) if kind == "fp8_block" else (M,), dtype=torch.float32,
                    device="cuda")
    h.quantize(Xd, Q, S, kind, x_dtype)
    torch.cuda.synchronize()
    return Q.cpu().numpy(), S.cpu().numpy()


def check_bitwise(Qg, Sg, Qr, Sr, what):
    Qr8 = np.ascontiguousarray(Qr).view(np.uint8)
    bad = np.argwhere(Qg != Qr8)
    assert bad.size == 0, f"{what}: {len(bad)} codes differ, first {bad[:4].tolist()} " \
                          f"got {[int(Qg[tuple(b)]) for b in bad[:4]]} want {[int(Qr8[tuple(b)]) for b in bad[:4]]}"
    assert np.array_equal(Sg.view(np.uint32), Sr.view(np.uint32)), f"{what}: scales differ"


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("x_dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("shape", SHAPES, ids=[f"{m}x{k}" for m, k in SHAPES])
def test_quantize_matches_oracle_bitwise(handle, kind, x_dtype, shape):
    M, K = shape
    if kind == "fp8_block" and K % 128:
        pytest.skip("1x128 blocks need K % 128 == 0")
    X = synth.activations16(M, K, seed=17 * M + K, x_dtype=x_dtype)
    print(f"[quant] {kind} {x_dtype} {M}x{K}", flush=True)
    Qr, Sr = oracle.dynamic_quant(kind, X, x_dtype)
    Qg, Sg = gpu_quantize(handle, X, kind, x_dtype)
    check_bitwise(Qg, Sg, Qr, Sr, f"{kind} {x_dtype} {M}x{K}")


def special_rows():
    """Rows whose scale is exactly 1: every e4m3 value, every midpoint
    between neighbours and the bf16 values beside each midpoint (row 0), int8
    halves (row 1), an all-zero row with a -0 (row 2), tiny and subnormal
    magnitudes (row 3)."""
    codes = np.arange(127, dtype=np.uint8)
    v = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    mid = ((v[:-1].astype(np.float64) + v[1:]) / 2).astype(np.float32)
    b = synth.to_bf16_bits(mid).astype(np.int32)
    beside = np.concatenate([b - 1, b + 1]).astype(np.uint16)
    row0 = np.concatenate([synth.to_bf16_bits(np.concatenate([v, mid, -v, -mid])),
                           beside, beside | 0x8000])
    K = ((row0.size + 127) // 128) * 128
    X = np.zeros((4, K), np.uint16)
    X[0, :row0.size] = row0
    halves = np.array([127, 2.5, 3.5, -2.5, -3.5, 0.5, -0.5, 126.5, 1.5, -1.5, 100.25,
                       -100.75], np.float32)
    X[1, :halves.size] = synth.to_bf16_bits(halves)
    X[2, 7] = 0x8000
    tiny = np.float32(2.0) ** -np.arange(5, 30, dtype=np.float32)
    X[3, :tiny.size] = synth.to_bf16_bits(tiny)
    X[3, tiny.size:2 * tiny.size] = synth.to_bf16_bits(-tiny)
    return X


@pytest.mark.parametrize("kind", KINDS)
def test_quantize_special_rows(handle, kind):
    X = special_rows()
    Qr, Sr = oracle.dynamic_quant(kind, X)
    Qg, Sg = gpu_quantize(handle, X, kind, "bf16")
    check_bitwise(Qg, Sg, Qr, Sr, f"special rows {kind}")


def test_quantize_zero_rows_is_a_noop(handle):
    Q = torch.full((1, 16), 7, dtype=torch.uint8, device="cuda")
    S = torch.full((1,), 3.0, dtype=torch.float32, device="cuda")
    X = torch.zeros((0, 16), dtype=torch.int16, device="cuda")
    handle.quantize(X, Q, S, "fp8_token")
    torch.cuda.synchronize()
    assert int(Q[0, 0]) == 7 and float(S[0]) == 3.0


# (quant, act, M, N, K, bias, residual): decode, tile and ping-pong families
DYN_CASES = [
    ("fp8_dynamic", "none", 1, 1040, 4096, True, False),
    ("fp8_dynamic", "gelu_tanh", 32, 512, 1024, True, True),
    ("fp8_dynamic", "silu", 40, 384, 512, False, False),
    ("w8a8_int8", "silu", 8, 2064, 4096, False, False),
    ("w8a8_int8", "none", 300, 512, 1024, True, False),
    ("block_fp8", "none", 4, 512, 3072, False, True),
    ("block_fp8", "gelu_tanh", 300, 256, 1024, True, False),
]


@pytest.mark.parametrize("case", DYN_CASES, ids=[f"{c[0]}-M{c[2]}-N{c[3]}-K{c[4]}" for c in DYN_CASES])
def test_run_dynamic_matches_oracle(handle, case):
    quant, act, M, N, K, b, r = case
    p = synth.make_custom(quant, act, M, N, K, seed=5 * M + N, bias=b, residual=r)
    X = synth.activations16(M, K, seed=3 * M + K)
    kind = {"fp8_dynamic": "fp8_token", "w8a8_int8": "int8_token", "block_fp8": "fp8_block"}[quant]
    Qr, Sr = oracle.dynamic_quant(kind, X)
    ref, acc = oracle.linear(quant, act, Qr, p.B, Sr, p.sb, p.bias, p.residual, p.alpha)
    print(f"[dyn] {quant} {act} {M}x{N}x{K} -> {handle.describe(quant, M, N, K)}", flush=True)
    C = torch.empty((M, N), dtype=torch.int16, device="cuda")
    handle.run_dynamic(dev(X), dev(p.B), C, quant=quant, act=act, sb=dev(p.sb), alpha=p.alpha,
                       bias=dev(p.bias), residual=dev(p.residual))
    torch.cuda.synchronize()
    assert_close(decode_out(C, quant), ref, f"run_dynamic {quant} {M}x{N}x{K}")
    if acc is not None:
        Craw = torch.empty((M, N), dtype=torch.int32, device="cuda")
        handle.run_dynamic(dev(X), dev(p.B), Craw, quant=quant, act="raw_acc", sb=dev(p.sb))
        torch.cuda.synchronize()
        assert np.array_equal(Craw.cpu().numpy(), acc), "int8 accumulator after dynamic quant"


def test_run_dynamic_staging_grows_and_shrinks(handle):
    # A large call then a small one on the same handle: the staging is reused.
    for M in (64, 3):
        p = synth.make_custom("fp8_dynamic", "none", M, 256, 512, seed=M, bias=True)
        X = synth.activations16(M, 512, seed=M + 1)
        Qr, Sr = oracle.dynamic_quant("fp8_token", X)
        ref, _ = oracle.linear("fp8_dynamic", "none", Qr, p.B, Sr, p.sb, p.bias)
        C = torch.empty((M, 256), dtype=torch.int16, device="cuda")
        handle.run_dynamic(dev(X), dev(p.B), C, quant="fp8_dynamic", sb=dev(p.sb),
                           bias=dev(p.bias))
        torch.cuda.synchronize()
        assert_close(decode_out(C, "fp8_dynamic"), ref, f"staging M={M}")


# The quantization prologue inside the decode kernel (lin_gemm_run_dynamic,
# bf16 activations, up to 16 tokens): each compiled prologue variant against
# the oracle, and bit for bit against the same variant fed by the separate
# quantization kernel (the default, dq=0): the codes, scales and summation
# order are the same, so the outputs must be identical.
DQ_SHAPES = [(8, 1, 12), (8, 2, 16), (8, 4, 12), (8, 4, 24), (12, 1, 16), (4, 4, 16)]
DQ_CASES = [
    ("fp8_dynamic", "none", 1, 1040, 4096, True, False),
    ("fp8_dynamic", "gelu_tanh", 5, 528, 272, True, True),
    ("fp8_dynamic", "silu", 16, 6144, 4096, True, False),
    ("w8a8_int8", "silu", 8, 2064, 4096, False, False),
    ("w8a8_int8", "none", 2, 256, 1040, True, True),
    ("block_fp8", "none", 3, 512, 3072, False, True),
    ("block_fp8", "gelu_tanh", 16, 256, 1024, True, False),
]


def _dyn_run(handle, X, p, spec, act=None, raw=False):
    M, N = p.M, p.N
    C = torch.empty((M, N), dtype=torch.int32 if raw else torch.int16, device="cuda")
    handle.set_force(spec)
    try:
        handle.run_dynamic(X, dev(p.B), C, quant=p.quant, act="raw_acc" if raw else (act or p.act),
                           sb=dev(p.sb), alpha=p.alpha, bias=dev(p.bias),
                           residual=dev(p.residual))
    finally:
        handle.set_force(None)
    torch.cuda.synchronize()
    return C.cpu()


@pytest.mark.parametrize("case", DQ_CASES, ids=[f"{c[0]}-M{c[2]}-N{c[3]}-K{c[4]}" for c in DQ_CASES])
def test_prologue_variants_match_oracle_and_two_kernel_path(handle, case):
    quant, act, M, N, K, b, r = case
    p = synth.make_custom(quant, act, M, N, K, seed=11 * M + K, bias=b, residual=r)
    Xh = synth.activations16(M, K, seed=7 * M + N)
    kind = {"fp8_dynamic": "fp8_token", "w8a8_int8": "int8_token", "block_fp8": "fp8_block"}[quant]
    Qr, Sr = oracle.dynamic_quant(kind, Xh)
    ref, acc = oracle.linear(quant, act, Qr, p.B, Sr, p.sb, p.bias, p.residual, p.alpha)
    X = dev(Xh)
    for w, u, rows in DQ_SHAPES:
        if quant == "block_fp8" and 128 % rows:
            continue
        spec = f"decode swap=1 split=1 reduce=twopass waves={w} unroll={u} rows={rows}"
        print(f"[prologue] {quant} {M}x{N}x{K} {spec}", flush=True)
        C1 = _dyn_run(handle, X, p, spec + " dq=1")
        assert_close(decode_out(C1, quant), ref, f"prologue {quant} {M}x{N}x{K} [{spec}]")
        C0 = _dyn_run(handle, X, p, spec)
        assert torch.equal(C1, C0), f"prologue vs two-kernel differ [{spec}]"
        if acc is not None:
            Craw = _dyn_run(handle, X, p, spec + " dq=1", raw=True)
            assert np.array_equal(Craw.numpy(), acc), f"int8 accumulator [{spec}]"


def test_prologue_falls_back_when_lds_does_not_fit(handle):
    # 16 tokens of K = 12288 codes need ~197 KB of LDS: the call takes the
    # two-kernel path and still matches the oracle.
    p = synth.make_custom("block_fp8", "none", 16, 256, 12288, seed=3, bias=True)
    Xh = synth.activations16(16, 12288, seed=4)
    Qr, Sr = oracle.dynamic_quant("fp8_block", Xh)
    ref, _ = oracle.linear("block_fp8", "none", Qr, p.B, Sr, p.sb, p.bias)
    C = _dyn_run(handle, dev(Xh), p, "decode swap=1 split=1 reduce=twopass waves=8 unroll=1 rows=16 dq=1")
    assert_close(decode_out(C, "block_fp8"), ref, "block fp8 16 x 12288 fallback")


# Fused quantization with widened activations ("xs=2 dq=1", e4m3 per token):
# every wave quantizes its K range after a workgroup-wide maximum and widens
# the codes once into LDS.  The codes, scales and summation order are those
# of the two-kernel path with the same variant, so the outputs must be
# identical bit for bit; also against the oracle.  Includes an all-zero
# token (scale 1), a token of tiny values (the rescaled division) and a
# ragged K tail.
QW_SHAPES = [(8, 2, 12), (8, 1, 12), (8, 4, 12), (12, 1, 16), (16, 1, 16), (8, 1, 24), (4, 4, 16)]
QW_CASES = [("none", 1, 1040, 4096, True, False), ("gelu_tanh", 3, 528, 272, True, True),
            ("silu", 5, 1040, 4096, False, True), ("none", 8, 6144, 4096, True, False),
            ("relu", 2, 272, 12304, True, False), ("none", 4, 256, 1024, False, False)]


@pytest.mark.parametrize("case", QW_CASES, ids=[f"M{c[1]}-N{c[2]}-K{c[3]}" for c in QW_CASES])
def test_fused_quantize_widen_matches_two_kernel_path(handle, case):
    act, M, N, K, b, r = case
    p = synth.make_custom("fp8_dynamic", act, M, N, K, seed=13 * M + K, bias=b, residual=r)
    Xh = synth.activations16(M, K, seed=5 * M + N)
    if M >= 3:
        Xh[1] = 0                                             # all-zero token
        tiny = (np.abs(Xh[2].view(np.int16).astype(np.int32)) & 0x7F) | 0x0100  # ~1e-37
        Xh[2] = (tiny | (Xh[2] & 0x8000)).astype(np.uint16)
    Qr, Sr = oracle.dynamic_quant("fp8_token", Xh)
    ref, _ = oracle.linear("fp8_dynamic", act, Qr, p.B, Sr, p.sb, p.bias, p.residual, p.alpha)
    X = dev(Xh)
    for w, u, rows in QW_SHAPES:
        spec = f"decode swap=1 split=1 reduce=twopass waves={w} unroll={u} rows={rows} xs=2"
        print(f"[qwiden] {M}x{N}x{K} {spec}", flush=True)
        C1 = _dyn_run(handle, X, p, spec + " dq=1")
        assert_close(decode_out(C1, "fp8_dynamic"), ref, f"fused {M}x{N}x{K} [{spec}]")
        C0 = _dyn_run(handle, X, p, spec)
        assert torch.equal(C1, C0), f"fused vs two-kernel differ [{spec}]"
        C2 = _dyn_run(handle, X, p, spec.replace(" xs=2", ""))
        assert torch.equal(C1, C2), f"fused vs plain variant differ [{spec}]"


@pytest.mark.parametrize("M", [1, 2])
def test_table_fused_quantization_at_decode_shape(handle, M):
    # The built-in table asks for the fused quantize-widen prologue for one
    # and two tokens at N = 6144, K = 4096: lin_gemm_run_dynamic through the
    # default dispatch against the oracle, and bit for bit against the same
    # variant fed by the separate quantization kernel.
    N, K = 6144, 4096
    desc = handle.describe("fp8_dynamic", M, N, K).split()
    assert "xs=2" in desc and "dq=1" in desc, desc
    p = synth.make_custom("fp8_dynamic", "silu", M, N, K, seed=17 + M, bias=True, residual=True)
    Xh = synth.activations16(M, K, seed=23 + M)
    Qr, Sr = oracle.dynamic_quant("fp8_token", Xh)
    ref, _ = oracle.linear("fp8_dynamic", "silu", Qr, p.B, Sr, p.sb, p.bias, p.residual, p.alpha)
    C = torch.empty((M, N), dtype=torch.int16, device="cuda")
    handle.run_dynamic(dev(Xh), dev(p.B), C, quant="fp8_dynamic", act="silu", sb=dev(p.sb),
                       alpha=p.alpha, bias=dev(p.bias), residual=dev(p.residual))
    torch.cuda.synchronize()
    assert_close(decode_out(C.cpu(), "fp8_dynamic"), ref, f"table fused M={M}")
    spec = handle.describe("fp8_dynamic", M, N, K).replace(" dq=1", "")
    C0 = _dyn_run(handle, dev(Xh), p, spec)
    assert torch.equal(C.cpu(), C0)
