"""Python binding of liblingemm.so, the MI355X scaled linear layer with a
fused epilogue (C ABI in include/lin_gemm.h).

Argument marshalling only: torch supplies device memory and the current HIP
stream; every step of the computation runs in the library's HIP kernels.
There is no CPU or PyTorch fallback -- if the library is not built, importing
works but every call raises.

    h = Handle()
    h.run(A, B, C, quant="fp8_dynamic", act="none", sa=sa, sb=sb, bias=bias)

PyTorch integration (custom operators with fake implementations, an FX pass
that fuses linear + epilogue chains) lives in ``epilogue_scaled_gemm_amd.torch_ops``.

Operands are contiguous CUDA tensors.  A[M,K] and B[N,K] hold bf16 / fp16 /
float8_e4m3fn / int8 values (or the same bytes as uint16 / uint8 views);
bias[N], residual[M,N] and C[M,N] are bf16 (fp16 in fp16 mode); sa, sb are
fp32 per the quant mode's layout (see the header).
"""
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblingemm.so")

QUANT = {"bf16": 0, "fp16": 1, "fp8_dynamic": 2, "w8a8_int8": 3, "block_fp8": 4, "mxfp4": 5}
ACT = {"none": 0, "relu": 1, "gelu_tanh": 2, "silu": 3, "raw_acc": 255}
STATUS = {0: "ok", -1: "invalid argument", -2: "unsupported", -3: "HIP error",
          -4: "out of memory", -5: "config error"}

# The symbols include/lin_gemm.h declares.
EXPORTS = ("lin_gemm_create", "lin_gemm_run", "lin_gemm_destroy", "lin_gemm_strerror",
           "lin_gemm_last_error", "lin_gemm_set_force", "lin_gemm_describe",
           "lin_gemm_run_unfused", "lin_gemm_quantize", "lin_gemm_run_dynamic",
           "lin_gemm_run_grouped", "lin_gemm_run_noalloc", "lin_gemm_stream_read")
DQ_KIND = {"fp8_token": 0, "int8_token": 1, "fp8_block": 2}
X_DTYPE = {"bf16": 0, "fp16": 1}


class LinGemmError(RuntimeError):
    def __init__(self, status, detail=""):
        self.status = status
        super().__init__(f"lin_gemm: {STATUS.get(status, status)} ({status}): {detail}")


class _Scales(ctypes.Structure):
    _fields_ = [("a", ctypes.c_void_p), ("b", ctypes.c_void_p), ("alpha", ctypes.c_float)]


_lib = None


def library():
    """Load liblingemm.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run `python -m epilogue_scaled_gemm_amd.build`"
                           " or __graft_entry__.build()")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    lib.lin_gemm_create.argtypes = [ctypes.POINTER(P), ctypes.c_char_p]
    lib.lin_gemm_create.restype = I
    lib.lin_gemm_run.argtypes = [P, P, P, ctypes.POINTER(_Scales), P, P, P, I64, I64, I64, I, I, P]
    lib.lin_gemm_run.restype = I
    lib.lin_gemm_run_noalloc.argtypes = lib.lin_gemm_run.argtypes
    lib.lin_gemm_run_noalloc.restype = I
    lib.lin_gemm_destroy.argtypes = [P]
    lib.lin_gemm_destroy.restype = I
    lib.lin_gemm_strerror.argtypes = [I]
    lib.lin_gemm_strerror.restype = ctypes.c_char_p
    lib.lin_gemm_last_error.argtypes = [P]
    lib.lin_gemm_last_error.restype = ctypes.c_char_p
    lib.lin_gemm_set_force.argtypes = [P, ctypes.c_char_p]
    lib.lin_gemm_set_force.restype = I
    lib.lin_gemm_describe.argtypes = [P, I, I64, I64, I64, ctypes.c_char_p, I]
    lib.lin_gemm_describe.restype = I
    lib.lin_gemm_run_unfused.argtypes = [P, P, P, P, P, P, P, P, I64, I64, I64, ctypes.c_float,
                                         I, I, P]
    lib.lin_gemm_run_unfused.restype = I
    lib.lin_gemm_stream_read.argtypes = [P, P, I64, I, I, P, P]
    lib.lin_gemm_stream_read.restype = I
    lib.lin_gemm_quantize.argtypes = [P, P, I, I64, I64, I, P, P, P]
    lib.lin_gemm_quantize.restype = I
    lib.lin_gemm_run_dynamic.argtypes = [P, P, I, P, P, ctypes.c_float, P, P, P, I64, I64, I64,
                                         I, I, P]
    lib.lin_gemm_run_dynamic.restype = I
    lib.lin_gemm_run_grouped.argtypes = [P, P, P, ctypes.POINTER(_Scales), P, P, P, P, I64, I64,
                                         I64, I64, I64, I, I, P]
    lib.lin_gemm_run_grouped.restype = I
    _lib = lib
    return lib


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _code(table, key):
    if isinstance(key, int):
        return key
    return table[key]


_QNAME = {v: k for k, v in QUANT.items()}


def _need(name, t, count, esize):
    """t must hold at least `count` elements of `esize` bytes: the kernels
    read that many from its address.  (The library sees only pointers, so
    these checks are the binding's part of argument marshalling.)"""
    if t is None or count <= 0:
        return
    if t.element_size() != esize:
        raise ValueError(f"{name}: elements must be {esize} bytes, got {t.dtype}")
    if t.numel() < count:
        raise ValueError(f"{name}: needs {count} elements, got {t.numel()} "
                         f"(shape {tuple(t.shape)}; no broadcasting)")


def _check_layer(quant, act, M, N, K, A=None, B=None, C=None, sa=None, sb=None, bias=None,
                 residual=None, a16=False):
    """Byte sizes of a layer call's operands (layouts of include/lin_gemm.h)."""
    q = _QNAME.get(quant, quant) if isinstance(quant, int) else quant
    a_es = 2 if (a16 or q in ("bf16", "fp16", "mxfp4")) else 1
    kb = K // 2 if q == "mxfp4" else K * (2 if q in ("bf16", "fp16") else 1)
    for name, t, nbytes in (("A", A, M * K * a_es), ("B", B, N * kb)):
        if t is not None and t.numel() * t.element_size() < nbytes:
            raise ValueError(f"{name}: needs {nbytes} bytes, got {t.numel() * t.element_size()}")
    raw = act in ("raw_acc", 255)
    _need("C", C, M * N, 4 if raw else 2)
    _need("bias", bias, N, 2)
    _need("residual", residual, M * N, 2)
    if q in ("fp8_dynamic", "w8a8_int8"):
        _need("sa", sa, M, 4)
        _need("sb", sb, N, 4)
    elif q == "block_fp8":
        _need("sa", sa, M * (K // 128), 4)
        _need("sb", sb, (N // 128) * (K // 128), 4)
    elif q == "mxfp4":
        _need("sb (E8M0 bytes)", sb, N * (K // 32), 1)


class Handle:
    """One lin_gemm handle (variant table + split-K workspace)."""

    def __init__(self, config_path=None):
        self._lib = library()
        h = ctypes.c_void_p()
        path = None if config_path is None else str(config_path).encode()
        rc = self._lib.lin_gemm_create(ctypes.byref(h), path)
        if rc != 0:
            raise LinGemmError(rc, f"lin_gemm_create({config_path!r})")
        self._h = h

    def _check(self, rc, what):
        if rc != 0:
            detail = self._lib.lin_gemm_last_error(self._h).decode(errors="replace")
            raise LinGemmError(rc, f"{what}: {detail}")

    def run(self, A, B, C, quant="bf16", act="none", sa=None, sb=None, alpha=1.0, bias=None,
            residual=None, stream=None, M=None, N=None, K=None):
        """C = act(scale(A B^T) + bias) * alpha + residual, on the current stream."""
        M = A.shape[0] if M is None else M
        K = A.shape[1] if K is None else K
        N = B.shape[0] if N is None else N
        kb = K // 2 if quant in ("mxfp4", 5) else K  # 4-bit weights: two codes per byte
        if B.shape[1] != kb:
            raise ValueError(f"inner dimensions differ: A has K={K}, B rows have {B.shape[1]}")
        _check_layer(quant, act, M, N, K, A, B, C, sa, sb, bias, residual)
        sc = _Scales(None if sa is None else _ptr(sa).value,
                     None if sb is None else _ptr(sb).value, float(alpha))
        rc = self._lib.lin_gemm_run(self._h, _ptr(A), _ptr(B), ctypes.byref(sc), _ptr(bias),
                                    _ptr(residual), _ptr(C), M, N, K, _code(QUANT, quant),
                                    _code(ACT, act), _stream(stream))
        self._check(rc, "lin_gemm_run")
        return C

    def run_unfused(self, A, B, C, T, U, quant="bf16", act="gelu_tanh", alpha=1.0, bias=None,
                    residual=None, stream=None):
        """The three-kernel unfused path (GEMM -> T, act(T + bias) -> U,
        alpha * U + residual -> C); measurement only."""
        M, K = A.shape
        N = B.shape[0]
        rc = self._lib.lin_gemm_run_unfused(self._h, _ptr(A), _ptr(B), _ptr(bias), _ptr(residual),
                                            _ptr(C), _ptr(T), _ptr(U), M, N, K, float(alpha),
                                            _code(QUANT, quant), _code(ACT, act), _stream(stream))
        self._check(rc, "lin_gemm_run_unfused")
        return C

    def stream_read(self, src, sink, grid=0, unroll=8, nbytes=None, stream=None):
        """Measurement only: a plain streaming read of src (its bytes, or the
        first nbytes); sink is an int32 CUDA tensor of at least 256 entries."""
        nb = src.numel() * src.element_size() if nbytes is None else int(nbytes)
        if nb > src.numel() * src.element_size():
            raise ValueError("nbytes beyond the tensor")
        _need("sink", sink, 256, 4)
        rc = self._lib.lin_gemm_stream_read(self._h, _ptr(src), nb, int(grid), int(unroll),
                                            _ptr(sink), _stream(stream))
        self._check(rc, "lin_gemm_stream_read")

    def quantize(self, X, Q, scales, kind="fp8_token", x_dtype="bf16", stream=None):
        """Dynamic activation quantization of X[M,K] into Q[M,K] and scales."""
        M, K = X.shape
        rc = self._lib.lin_gemm_quantize(self._h, _ptr(X), _code(X_DTYPE, x_dtype), M, K,
                                         _code(DQ_KIND, kind), _ptr(Q), _ptr(scales),
                                         _stream(stream))
        self._check(rc, "lin_gemm_quantize")
        return Q, scales

    def run_dynamic(self, X, B, C, quant="fp8_dynamic", act="none", sb=None, alpha=1.0,
                    bias=None, residual=None, x_dtype="bf16", stream=None):
        """Quantize X[M,K] (16-bit) on the fly, then the layer of run()."""
        M, K = X.shape
        N = B.shape[0]
        if B.shape[1] != K:
            raise ValueError(f"inner dimensions differ: X has K={K}, B has {B.shape[1]}")
        _check_layer(quant, act, M, N, K, X, B, C, None, sb, bias, residual, a16=True)
        rc = self._lib.lin_gemm_run_dynamic(self._h, _ptr(X), _code(X_DTYPE, x_dtype), _ptr(B),
                                            _ptr(sb), float(alpha), _ptr(bias), _ptr(residual),
                                            _ptr(C), M, N, K, _code(QUANT, quant),
                                            _code(ACT, act), _stream(stream))
        self._check(rc, "lin_gemm_run_dynamic")
        return C

    def run_grouped(self, A, B, C, offsets, quant="bf16", act="none", sa=None, sb=None,
                    alpha=1.0, bias=None, residual=None, max_rows=0, stream=None):
        """Mixture-of-experts layer: A[M,K] rows sorted by expert, B[E,N,K]
        (E,N,K/2 bytes for mxfp4), offsets int32[E+1] on the GPU; expert x's
        rows [offsets[x], offsets[x+1]) use B[x], sb[x] and bias[x]."""
        M, K = A.shape
        E, N, kb = B.shape
        if kb != (K // 2 if quant in ("mxfp4", 5) else K):
            raise ValueError(f"inner dimensions differ: A has K={K}, B rows have {kb}")
        if offsets.dtype != torch.int32 or offsets.numel() != E + 1:
            raise ValueError("offsets must be int32 with E + 1 entries")
        sc = _Scales(None if sa is None else _ptr(sa).value,
                     None if sb is None else _ptr(sb).value, float(alpha))
        rc = self._lib.lin_gemm_run_grouped(self._h, _ptr(A), _ptr(B), ctypes.byref(sc),
                                            _ptr(bias), _ptr(residual), _ptr(C), _ptr(offsets),
                                            E, M, N, K, int(max_rows), _code(QUANT, quant),
                                            _code(ACT, act), _stream(stream))
        self._check(rc, "lin_gemm_run_grouped")
        return C

    def set_force(self, spec):
        rc = self._lib.lin_gemm_set_force(self._h, None if not spec else spec.encode())
        self._check(rc, f"lin_gemm_set_force({spec!r})")

    def describe(self, quant, M, N, K):
        buf = ctypes.create_string_buffer(256)
        rc = self._lib.lin_gemm_describe(self._h, _code(QUANT, quant), M, N, K, buf, 256)
        self._check(rc, "lin_gemm_describe")
        return buf.value.decode()

    def close(self):
        if getattr(self, "_h", None):
            self._lib.lin_gemm_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


def strerror(status):
    return library().lin_gemm_strerror(status).decode()


def out_dtype(quant):
    return torch.float16 if quant in ("fp16", 1) else torch.bfloat16
