"""CPU oracle for the scaled linear layer with a fused epilogue.

TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check in __graft_entry__ and
the benchmark's cpu_baseline leg may import this package.  The product path
(the HIP library and its Python binding) never touches it, and the two share
no code: they meet only at the raw byte arrays produced by the seeded input
generators in ``synth``.

The arithmetic lives in oracle.c (plain C, fp64 / int64, exact decoders); this
module is argument marshalling over ctypes plus numpy-shaped convenience
wrappers.  See oracle.c for the definition and the passages it follows.

Parity pins (tests/test_oracle_*.py): exhaustive e4m3 decode against torch's
CPU cast, bf16/fp16 decode and bf16 rounding against torch/numpy casts, exact
Fraction brute force on tiny shapes for every quant mode (epilogue through
torch's fp64 activations), the activations against torch's own fp64
gelu(approximate="tanh") / silu / relu on a dense grid, the listing's two GELU
constants recovered from the oracle's outputs, the SiLU logit identity and the
odd-part identity, identity and permutation
weights, the block-scale closed form, the transpose (swap-AB) identity, and
the 32 MiB size of a 4096x4096 16-bit intermediate; for the dynamic
quantization, every e4m3 code and every midpoint between neighbours against
torch's CPU cast, int8 ties-to-even on exact halves, the group maximum mapping
to the format's maximum, the half-step error bound, and the block kind equal to
the per-token kind over 128-wide rows.  Unpinned: nothing in the
oracle itself; the GPU's fp32 accumulation order is covered only by the
stated tolerance.
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")

QUANT = {"bf16": 0, "fp16": 1, "fp8_dynamic": 2, "w8a8_int8": 3, "block_fp8": 4, "mxfp4": 5}
ACT = {"none": 0, "relu": 1, "gelu_tanh": 2, "silu": 3}

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.oracle_e4m3_to_f64.restype = ctypes.c_double
    lib.oracle_e4m3_to_f64.argtypes = [ctypes.c_uint8]
    lib.oracle_bf16_to_f64.restype = ctypes.c_double
    lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_fp16_to_f64.restype = ctypes.c_double
    lib.oracle_fp16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_e2m1_to_f64.restype = ctypes.c_double
    lib.oracle_e2m1_to_f64.argtypes = [ctypes.c_uint8]
    lib.oracle_e8m0_to_f64.restype = ctypes.c_double
    lib.oracle_e8m0_to_f64.argtypes = [ctypes.c_uint8]
    lib.oracle_f64_to_bf16_rne.restype = ctypes.c_uint16
    lib.oracle_f64_to_bf16_rne.argtypes = [ctypes.c_double]
    lib.oracle_act.restype = ctypes.c_double
    lib.oracle_act.argtypes = [ctypes.c_int, ctypes.c_double]
    lib.oracle_linear.restype = ctypes.c_int
    lib.oracle_linear.argtypes = [P, P, P, P, ctypes.c_double, P, P, I64, I64, I64,
                                  ctypes.c_int, ctypes.c_int, P, P, ctypes.c_int]
    lib.oracle_linear_at.restype = ctypes.c_int
    lib.oracle_linear_at.argtypes = [P, P, P, P, ctypes.c_double, P, P, I64, I64, I64,
                                     ctypes.c_int, ctypes.c_int, P, P, I64, P, P,
                                     ctypes.c_int]
    lib.oracle_unfused_stage2.restype = ctypes.c_int
    lib.oracle_unfused_stage2.argtypes = [P, P, I64, I64, ctypes.c_int, ctypes.c_int, P]
    lib.oracle_unfused_stage3.restype = ctypes.c_int
    lib.oracle_unfused_stage3.argtypes = [P, P, ctypes.c_double, I64, I64, ctypes.c_int, P]
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_f32_to_e4m3_rne.restype = ctypes.c_uint8
    lib.oracle_f32_to_e4m3_rne.argtypes = [ctypes.c_float]
    lib.oracle_dynamic_quant.restype = ctypes.c_int
    lib.oracle_dynamic_quant.argtypes = [P, I64, I64, ctypes.c_int, ctypes.c_int, P, P]
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def e4m3_to_f64(code: int) -> float:
    return _load().oracle_e4m3_to_f64(code)


def bf16_to_f64(bits: int) -> float:
    return _load().oracle_bf16_to_f64(bits)


def fp16_to_f64(bits: int) -> float:
    return _load().oracle_fp16_to_f64(bits)


def e2m1_to_f64(code: int) -> float:
    return _load().oracle_e2m1_to_f64(code)


def e8m0_to_f64(code: int) -> float:
    return _load().oracle_e8m0_to_f64(code)


def f64_to_bf16(x: float) -> int:
    return _load().oracle_f64_to_bf16_rne(x)


def act(name: str, y: float) -> float:
    return _load().oracle_act(ACT[name], y)


def num_threads() -> int:
    return _load().oracle_num_threads()


def _operands(quant, A, B, sa, sb, bias, residual):
    q = QUANT[quant]
    if q == 5:  # bf16 activations, packed E2M1 weights, E8M0 weight scales
        return q, _c(A, np.uint16), _c(B, np.uint8), None, _c(sb, np.uint8), \
            _c(bias, np.uint16), _c(residual, np.uint16)
    code_t = np.uint16 if q in (0, 1) else (np.int8 if q == 3 else np.uint8)
    A = _c(A, code_t)
    B = _c(B, code_t)
    sa = _c(sa, np.float32)
    sb = _c(sb, np.float32)
    bias = _c(bias, np.uint16)
    residual = _c(residual, np.uint16)
    return q, A, B, sa, sb, bias, residual


_ERR = {-1: "invalid argument", -2: "int8 accumulator overflows int32"}


def linear(quant, act_name, A, B, sa=None, sb=None, bias=None, residual=None, alpha=1.0,
           nthreads=0):
    """Reference result r[M,N] (fp64) and, for int8, the int32 accumulator.

    A: [M,K] codes, B: [N,K] codes (uint16 for bf16/fp16, uint8 for e4m3,
    int8 for int8; for mxfp4 [N,K/2] bytes of two E2M1 codes, low nibble
    first).  sa/sb fp32 per the quant mode's layout (mxfp4: sb is E8M0
    bytes [N,K/32], sa unused).  bias [N] and
    residual [M,N] are 16-bit float codes.  Returns (r, acc or None).
    """
    q, A, B, sa, sb, bias, residual = _operands(quant, A, B, sa, sb, bias, residual)
    M, K = A.shape
    N = B.shape[0]
    assert B.shape[1] == (K // 2 if q == 5 else K)
    out = np.empty((M, N), dtype=np.float64)
    acc = np.zeros((M, N), dtype=np.int32) if q == 3 else None
    rc = _load().oracle_linear(_ptr(A), _ptr(B), _ptr(sa), _ptr(sb), float(alpha),
                               _ptr(bias), _ptr(residual), M, N, K, q, ACT[act_name],
                               _ptr(out), _ptr(acc), int(nthreads))
    if rc:
        raise ValueError(f"oracle_linear: {_ERR.get(rc, rc)}")
    return out, acc


def linear_at(quant, act_name, A, B, idx_m, idx_n, sa=None, sb=None, bias=None,
              residual=None, alpha=1.0, nthreads=0):
    """Reference values at the positions (idx_m[i], idx_n[i]) only."""
    q, A, B, sa, sb, bias, residual = _operands(quant, A, B, sa, sb, bias, residual)
    M, K = A.shape
    N = B.shape[0]
    im = _c(idx_m, np.int64)
    inn = _c(idx_n, np.int64)
    cnt = im.shape[0]
    out = np.empty(cnt, dtype=np.float64)
    acc = np.zeros(cnt, dtype=np.int32) if q == 3 else None
    rc = _load().oracle_linear_at(_ptr(A), _ptr(B), _ptr(sa), _ptr(sb), float(alpha),
                                  _ptr(bias), _ptr(residual), M, N, K, q, ACT[act_name],
                                  _ptr(im), _ptr(inn), cnt, _ptr(out), _ptr(acc),
                                  int(nthreads))
    if rc:
        raise ValueError(f"oracle_linear_at: {_ERR.get(rc, rc)}")
    return out, acc


def grouped_linear(quant, act_name, A, Bs, offsets, sa=None, sbs=None, biases=None,
                   residual=None, alpha=1.0):
    """Grouped layer (a mixture-of-experts linear): tokens sorted by expert,
    expert e owning the rows [offsets[e], offsets[e+1]) of A, residual and the
    result, multiplied by its own weight Bs[e] with its own weight scales
    sbs[e] and bias biases[e].  Each segment is exactly `linear` on its rows;
    per-token activation scales sa are sliced with the rows.  Returns the
    [M, N] result and, for int8, the accumulator.

    "helion-vllm-linear-backend", section "Что дальше": a mixture-of-experts
    backend is named as work in progress and not defined; this is the plain
    reading (a per-expert product over each expert's rows)."""
    M = A.shape[0]
    N = Bs[0].shape[0]
    out = np.zeros((M, N), dtype=np.float64)
    acc = np.zeros((M, N), dtype=np.int32) if quant == "w8a8_int8" else None
    for e in range(len(Bs)):
        m0, m1 = int(offsets[e]), int(offsets[e + 1])
        if m1 <= m0:
            continue
        r, a = linear(quant, act_name, A[m0:m1], Bs[e],
                      None if sa is None else sa[m0:m1],
                      None if sbs is None else sbs[e],
                      None if biases is None else biases[e],
                      None if residual is None else residual[m0:m1], alpha)
        out[m0:m1] = r
        if acc is not None:
            acc[m0:m1] = a
    return out, acc


def unfused_stage2(t, bias, quant="bf16", act_name="gelu_tanh"):
    t = _c(t, np.uint16)
    M, N = t.shape
    u = np.empty((M, N), dtype=np.float64)
    _load().oracle_unfused_stage2(_ptr(t), _ptr(_c(bias, np.uint16)), M, N, QUANT[quant],
                                  ACT[act_name], _ptr(u))
    return u


def unfused_stage3(u, residual, alpha, quant="bf16"):
    u = _c(u, np.uint16)
    M, N = u.shape
    o = np.empty((M, N), dtype=np.float64)
    _load().oracle_unfused_stage3(_ptr(u), _ptr(_c(residual, np.uint16)), float(alpha), M, N,
                                  QUANT[quant], _ptr(o))
    return o


DQ_KIND = {"fp8_token": 0, "int8_token": 1, "fp8_block": 2}


def f32_to_e4m3(v: float) -> int:
    """E4M3FN code nearest to the binary32 value v (ties to even, saturating)."""
    return _load().oracle_f32_to_e4m3_rne(v)


def dynamic_quant(kind, X, x_dtype="bf16"):
    """Dynamic activation quantization of X[M,K] (16-bit float codes).

    kind: "fp8_token" (e4m3 codes, scales [M]), "int8_token" (int8, [M]) or
    "fp8_block" (e4m3, scales [M, K/128]).  Returns (Q codes [M,K], scales).
    """
    X = _c(X, np.uint16)
    M, K = X.shape
    q_t = np.int8 if kind == "int8_token" else np.uint8
    Q = np.empty((M, K), dtype=q_t)
    sc = np.empty((M, K // 128) if kind == "fp8_block" else (M,), dtype=np.float32)
    rc = _load().oracle_dynamic_quant(_ptr(X), M, K, 1 if x_dtype == "fp16" else 0,
                                      DQ_KIND[kind], _ptr(Q), _ptr(sc))
    if rc:
        raise ValueError(f"oracle_dynamic_quant: {_ERR.get(rc, rc)}")
    return Q, sc


def within_tolerance(g, r, rel=1e-2, floor=1e-3):
    """The elementwise pass rule |g - r| <= rel * max(|r|, floor)."""
    g = np.asarray(g, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    return np.abs(g - r) <= rel * np.maximum(np.abs(r), floor)
