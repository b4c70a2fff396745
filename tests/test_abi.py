"""The C ABI: the library loads and exports every symbol include/lin_gemm.h
declares; the variant table parses; argument errors return the documented
status codes before anything reaches the GPU.

The CPU tests here never launch a kernel: every call either fails validation
or has M == 0.  Calls that would pass validation are only made in the GPU
tests, with real device tensors.
"""
import ctypes
import os
import re
import subprocess

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lin_gemm.h")

lg = pytest.importorskip("epilogue_scaled_gemm_amd")
pytestmark = pytest.mark.skipif(not os.path.exists(lg.LIB_PATH), reason="library not built")

OK, INVALID, UNSUPPORTED, CONFIG = 0, -1, -2, -5


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(lin_gemm_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    assert set(declared_functions()) == set(lg.EXPORTS)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", lg.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    syms = {l.split()[-1] for l in out.splitlines() if " T " in l}
    missing = [f for f in declared_functions() if f not in syms]
    assert not missing, missing
    lib = ctypes.CDLL(lg.LIB_PATH)
    for f in declared_functions():
        assert hasattr(lib, f)


def test_strerror():
    assert lg.strerror(0) == "ok"
    assert "invalid" in lg.strerror(-1)
    assert "unsupported" in lg.strerror(-2)


FAKE = 0x10000  # never dereferenced: every call below fails validation first


def _raw_run(h, A=FAKE, B=FAKE, C=FAKE, M=4, N=16, K=64, quant=0, act=0, scales=None,
             bias=None, residual=None):
    lib = lg.library()
    sc = lg._Scales(*(scales if scales else (None, None, 1.0)))
    return lib.lin_gemm_run(h._h, A, B, ctypes.byref(sc), bias, residual, C, M, N, K, quant, act,
                            None)


@pytest.fixture()
def cpu_handle():
    if torch.cuda.is_available():
        pytest.skip("fake-pointer error paths run on the CPU only")
    h = lg.Handle()
    yield h
    h.close()


@pytest.mark.parametrize("kw,status", [
    (dict(quant=7), INVALID),
    (dict(act=9), INVALID),
    (dict(M=-1), INVALID),
    (dict(A=None), INVALID),
    (dict(C=None), INVALID),
    (dict(quant=2), INVALID),                              # fp8 without scales
    (dict(quant=3, scales=(FAKE, None, 1.0)), INVALID),     # int8 missing sb
    (dict(K=60), UNSUPPORTED),                             # bf16 rows not 16-byte multiples
    (dict(quant=2, K=40, scales=(FAKE, FAKE, 1.0)), UNSUPPORTED),
    (dict(quant=4, N=100, K=256, scales=(FAKE, FAKE, 1.0)), UNSUPPORTED),
    (dict(quant=4, N=128, K=200, scales=(FAKE, FAKE, 1.0)), UNSUPPORTED),
    (dict(quant=3, K=131072, scales=(FAKE, FAKE, 1.0)), UNSUPPORTED),
    (dict(N=0), UNSUPPORTED),
    (dict(A=FAKE + 4), UNSUPPORTED),                       # misaligned
])
def test_argument_errors(cpu_handle, kw, status):
    assert _raw_run(cpu_handle, **kw) == status
    if status != OK:
        assert lg.library().lin_gemm_last_error(cpu_handle._h)


def test_zero_m_returns_ok_without_work(cpu_handle):
    assert _raw_run(cpu_handle, M=0) == OK


def test_force_and_describe(cpu_handle):
    h = cpu_handle
    assert h.describe("fp8_dynamic", 8, 6144, 4096).startswith("decode")
    assert h.describe("bf16", 4096, 4096, 4096).startswith("pp")
    h.set_force("decode swap=0 split=4 reduce=twopass waves=8 unroll=2")
    assert h.describe("w8a8_int8", 4, 24576, 4096) == \
        "decode swap=0 split=4 reduce=twopass waves=8 unroll=2 rows=16"
    with pytest.raises(lg.LinGemmError):
        h.describe("bf16", 64, 128, 128)          # forced decode with M > 32
    with pytest.raises(lg.LinGemmError):
        h.set_force("tile bm=96 bn=96 wm=2 wn=2")  # not a compiled shape
    with pytest.raises(lg.LinGemmError):
        h.set_force("decode split=3")              # not a power of two
    # auto split (split=0): 384 row groups of 16 -> 2 slices; 1536 -> 1
    h.set_force("decode swap=1 split=0 reduce=twopass waves=4 unroll=4 rows=16")
    assert "split=2" in h.describe("fp8_dynamic", 1, 6144, 4096)
    assert "split=1" in h.describe("w8a8_int8", 1, 24576, 4096)
    h.set_force(None)


def test_pp_force_and_split(cpu_handle):
    h = cpu_handle
    # block FP8 auto split: 256x128 tiles, slices doubled while the grid is
    # under 256 workgroups and each slice keeps >= 8 of the 96 scale blocks
    h.set_force("pp")
    assert h.describe("block_fp8", 512, 4096, 12288) == "pp split=4 group=4"
    assert h.describe("block_fp8", 2048, 4096, 12288) == "pp split=1 group=4"
    assert h.describe("block_fp8", 40, 4096, 12288) == "pp split=8 group=4"
    assert h.describe("bf16", 4096, 4096, 4096) == "pp split=1 group=4"
    assert h.describe("w8a8_int8", 300, 512, 1024) == "pp split=1 group=4"
    with pytest.raises(lg.LinGemmError):
        h.describe("fp8_dynamic", 512, 4096, 4096)   # no ping-pong kernel for per-channel e4m3
    # an explicit split is clamped to the number of scale blocks
    h.set_force("pp split=16")
    assert h.describe("block_fp8", 256, 512, 512) == "pp split=4 group=4"
    with pytest.raises(lg.LinGemmError):
        h.describe("bf16", 4096, 4096, 4096)         # split-K is for block FP8 only
    with pytest.raises(lg.LinGemmError):
        h.set_force("pp split=3")                    # not a power of two
    with pytest.raises(lg.LinGemmError):
        h.set_force("pp split=32")                   # beyond 16
    h.set_force(None)


def test_table_file(tmp_path):
    good = tmp_path / "t.cfg"
    good.write_text("# test table\nfp8_dynamic 1 32 6144 4096 decode swap=1 split=8 "
                    "reduce=atomic waves=8 unroll=1 rows=64\n* 1 * * * tile bm=64 bn=64 wm=2 wn=2\n")
    h = lg.Handle(str(good))
    assert h.describe("fp8_dynamic", 3, 6144, 4096) == \
        "decode swap=1 split=8 reduce=atomic waves=8 unroll=1 rows=64"
    assert h.describe("fp8_dynamic", 3, 6144, 8192).startswith("tile bm=64 bn=64")
    h.close()
    bad = tmp_path / "bad.cfg"
    bad.write_text("fp8_dynamic 1 64 * * decode swap=1\n")   # decode beyond 32 tokens
    with pytest.raises(lg.LinGemmError):
        lg.Handle(str(bad))
    with pytest.raises(lg.LinGemmError):
        lg.Handle(str(tmp_path / "missing.cfg"))


def test_built_in_table_parses_as_a_text_table(tmp_path, cpu_handle):
    # The sweep-written entries compiled into the library (csrc/table_mi355x.inc)
    # load through lin_gemm_create as a text table too, and every entry is
    # what lin_gemm_describe reports for its first token count.
    inc = os.path.join(os.path.dirname(lg.__file__), "csrc", "table_mi355x.inc")
    text = open(inc).read()
    body = text.split('R"TABLE(', 1)[1].split(')TABLE"', 1)[0]
    cfg = tmp_path / "table.cfg"
    cfg.write_text(body)
    h = lg.Handle(str(cfg))
    try:
        n = 0
        for line in body.splitlines():
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            q, lo, hi, N, K, *spec = line.split()
            got = h.describe(q, int(lo), int(N), int(K))
            want = " ".join(spec)
            # describe drops staging / prefetching where the shape cannot use
            # it and prints the split it resolves to; the kernel family and
            # the launch shape must match.
            assert got.split()[0] == want.split()[0]
            for key in ("waves", "unroll", "rows", "bm", "bn"):
                if f"{key}=" in want:
                    assert f"{key}={want.split(key + '=')[1].split()[0]}" in got, (line, got)
            n += 1
        assert n > 10
    finally:
        h.close()


def _raw_quantize(h, X=FAKE, x_dtype=0, M=4, K=256, kind=0, Q=FAKE, S=FAKE):
    return lg.library().lin_gemm_quantize(h._h, X, x_dtype, M, K, kind, Q, S, None)


@pytest.mark.parametrize("kw,status", [
    (dict(kind=3), INVALID),
    (dict(kind=-1), INVALID),
    (dict(x_dtype=2), INVALID),
    (dict(M=-1), INVALID),
    (dict(X=None), INVALID),
    (dict(Q=None), INVALID),
    (dict(S=None), INVALID),
    (dict(K=40), UNSUPPORTED),                 # not a multiple of 16
    (dict(K=0), UNSUPPORTED),
    (dict(kind=2, K=144), UNSUPPORTED),        # 1x128 blocks need K % 128
    (dict(X=FAKE + 8), UNSUPPORTED),           # misaligned
    (dict(Q=FAKE + 4), UNSUPPORTED),
    (dict(M=0), OK),                           # no-op
])
def test_quantize_argument_errors(cpu_handle, kw, status):
    assert _raw_quantize(cpu_handle, **kw) == status


@pytest.mark.parametrize("quant,status", [(0, INVALID), (1, INVALID), (5, INVALID)])
def test_run_dynamic_needs_a_quantised_mode(cpu_handle, quant, status):
    lib = lg.library()
    assert lib.lin_gemm_run_dynamic(cpu_handle._h, FAKE, 0, FAKE, FAKE, 1.0, None, None, FAKE,
                                    4, 16, 64, quant, 0, None) == status


def test_run_dynamic_shape_errors(cpu_handle):
    lib = lg.library()
    # e4m3 rows of 40 bytes; block FP8 with N % 128 != 0; null sb; M == 0
    assert lib.lin_gemm_run_dynamic(cpu_handle._h, FAKE, 0, FAKE, FAKE, 1.0, None, None, FAKE,
                                    4, 16, 40, 2, 0, None) == UNSUPPORTED
    assert lib.lin_gemm_run_dynamic(cpu_handle._h, FAKE, 0, FAKE, FAKE, 1.0, None, None, FAKE,
                                    4, 100, 256, 4, 0, None) == UNSUPPORTED
    assert lib.lin_gemm_run_dynamic(cpu_handle._h, FAKE, 0, FAKE, None, 1.0, None, None, FAKE,
                                    4, 16, 64, 2, 0, None) == INVALID
    assert lib.lin_gemm_run_dynamic(cpu_handle._h, FAKE, 0, FAKE, FAKE, 1.0, None, None, FAKE,
                                    0, 16, 64, 2, 0, None) == OK


@pytest.mark.parametrize("kw,status", [
    (dict(quant=5, K=640, scales=(None, FAKE, 1.0)), UNSUPPORTED),   # K % 256
    (dict(quant=5, M=33, K=512, scales=(None, FAKE + 4, 1.0)), UNSUPPORTED),  # misaligned
    (dict(quant=5, K=512, scales=(None, None, 1.0)), INVALID),       # no E8M0 scales
    (dict(quant=5, M=0, K=512, scales=(None, FAKE, 1.0)), OK),
])
def test_mxfp4_argument_errors(cpu_handle, kw, status):
    assert _raw_run(cpu_handle, **kw) == status


def test_mxfp4_describe(cpu_handle):
    v = cpu_handle.describe("mxfp4", 8, 6144, 4096)
    assert v.startswith("decode swap=1")
    for M in (33, 300, 4096):  # tile shapes whose weight loads split evenly
        v = dict(kv.split("=") for kv in cpu_handle.describe("mxfp4", M, 6144, 4096).split()[1:])
        assert int(v["bn"]) % (32 * int(v["wm"]) * int(v["wn"])) == 0, v
    cpu_handle.set_force("tile bm=64 bn=64 wm=2 wn=2")
    with pytest.raises(lg.LinGemmError):
        cpu_handle.describe("mxfp4", 64, 6144, 4096)
    cpu_handle.set_force(None)
    cpu_handle.set_force("decode swap=1 split=1 reduce=twopass waves=4 unroll=4 rows=16")
    with pytest.raises(lg.LinGemmError):
        cpu_handle.describe("mxfp4", 8, 6144, 4096)        # not compiled for MXFP4
    cpu_handle.set_force(None)


def _raw_grouped(h, A=FAKE, B=FAKE, C=FAKE, offsets=FAKE, E=4, M=8, N=16, K=64, max_rows=0,
                 quant=0, act=0, scales=None, bias=None, residual=None):
    lib = lg.library()
    sc = lg._Scales(*(scales if scales else (None, None, 1.0)))
    return lib.lin_gemm_run_grouped(h._h, A, B, ctypes.byref(sc), bias, residual, C, offsets, E,
                                    M, N, K, max_rows, quant, act, None)


@pytest.mark.parametrize("kw,status", [
    (dict(E=-1), INVALID),
    (dict(M=-1), INVALID),
    (dict(max_rows=-2), INVALID),
    (dict(quant=9), INVALID),
    (dict(act=7), INVALID),
    (dict(offsets=None), INVALID),
    (dict(A=None), INVALID),
    (dict(quant=2), INVALID),                                        # no scales
    (dict(quant=5, K=512, scales=(None, None, 1.0)), INVALID),       # no E8M0 scales
    (dict(K=20), UNSUPPORTED),                                       # 40-byte rows
    (dict(quant=4, N=100, K=256, scales=(FAKE, FAKE, 1.0)), UNSUPPORTED),
    (dict(quant=5, K=640, scales=(None, FAKE, 1.0)), UNSUPPORTED),   # K % 256
    (dict(E=70000), UNSUPPORTED),
    (dict(offsets=FAKE + 2), UNSUPPORTED),                           # misaligned offsets
    (dict(C=FAKE + 8), UNSUPPORTED),
    (dict(M=0), OK),                                                 # no-ops
    (dict(E=0), OK),
])
def test_grouped_argument_errors(cpu_handle, kw, status):
    assert _raw_grouped(cpu_handle, **kw) == status


@pytest.mark.parametrize("bad", ["residual_row", "residual_fp32", "bias_fp32", "sa_short",
                                 "C_short", "B_short"])
def test_binding_rejects_undersized_operands(bad):
    # The binding checks byte sizes before calling the library (which sees
    # only pointers); CPU tensors suffice since nothing is launched.
    M, N, K = 4, 32, 64
    t = dict(A=torch.zeros(M, K, dtype=torch.uint8), B=torch.zeros(N, K, dtype=torch.uint8),
             C=torch.zeros(M, N, dtype=torch.int16), sa=torch.ones(M), sb=torch.ones(N),
             bias=torch.zeros(N, dtype=torch.bfloat16),
             residual=torch.zeros(M, N, dtype=torch.bfloat16))
    if bad == "residual_row":
        t["residual"] = torch.zeros(N, dtype=torch.bfloat16)
    elif bad == "residual_fp32":
        t["residual"] = torch.zeros(M, N, dtype=torch.float32)
    elif bad == "bias_fp32":
        t["bias"] = torch.zeros(N, dtype=torch.float32)
    elif bad == "sa_short":
        t["sa"] = torch.ones(1)
    elif bad == "C_short":
        t["C"] = torch.zeros(M - 1, N, dtype=torch.int16)
    elif bad == "B_short":
        t["B"] = torch.zeros(N - 1, K, dtype=torch.uint8)
    with pytest.raises(ValueError):
        lg._check_layer("fp8_dynamic", "none", M, N, K, t["A"], t["B"], t["C"], t["sa"], t["sb"],
                        t["bias"], t["residual"])
    # the same operands with nothing wrong pass
    good = dict(A=torch.zeros(M, K, dtype=torch.uint8), B=torch.zeros(N, K, dtype=torch.uint8),
                C=torch.zeros(M, N, dtype=torch.int16), sa=torch.ones(M), sb=torch.ones(N),
                bias=torch.zeros(N, dtype=torch.bfloat16),
                residual=torch.zeros(M, N, dtype=torch.bfloat16))
    lg._check_layer("fp8_dynamic", "none", M, N, K, *good.values())
