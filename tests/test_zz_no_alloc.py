"""lin_gemm_run_noalloc: the entry point for callers that cannot allocate.

Called through the C ABI (ctypes on the library's own symbol) and checked
against lin_gemm_run on the same handle, variant and inputs: the same
kernels run, so deterministic reductions must give the same bits, int8
accumulators must be equal, and every floating-point output must also meet
the oracle's pass rule.  Each case makes two calls in a row, the second on a
smaller input, because every call on a device shares the one static scratch
array and keeps the last call's contents there.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_close, decode_out, out_tensor, reference, sample_positions, upload

pytestmark = pytest.mark.gpu

lg = pytest.importorskip("epilogue_scaled_gemm_amd")

UNSUPPORTED = -2


@pytest.fixture(scope="module")
def handle():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    h = lg.Handle()
    yield h
    h.set_force(None)
    h.close()


def _call(h, entry, p, d, C, raw=False):
    lib = lg.library()
    fn = lib.lin_gemm_run_noalloc if entry == "noalloc" else lib.lin_gemm_run
    sc = lg._Scales(None if d["sa"] is None else d["sa"].data_ptr(),
                    None if d["sb"] is None else d["sb"].data_ptr(), float(p.alpha))
    ptr = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())  # noqa: E731
    rc = fn(h._h, ptr(d["A"]), ptr(d["B"]), ctypes.byref(sc), ptr(d["bias"]),
            ptr(d["residual"]), ptr(C), p.M, p.N, p.K, lg.QUANT[p.quant],
            lg.ACT["raw_acc"] if raw else lg.ACT[p.act],
            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return rc


def _check_pair(h, p, force=None, raw=False, sampled=False, tag=""):
    """noalloc vs lin_gemm_run on p (same forced variant), then vs the oracle."""
    h.set_force(force)
    d = upload(p)
    print(f"[noalloc] {tag} {p.name} {p.M}x{p.N}x{p.K} "
          f"variant={h.describe(p.quant, p.M, p.N, p.K)}", flush=True)
    C_ref = out_tensor(p, raw)
    C_na = out_tensor(p, raw)
    C_na.fill_(0x7777 if C_na.dtype == torch.int16 else 7)
    assert _call(h, "run", p, d, C_ref, raw) == 0, lg.library().lin_gemm_last_error(h._h)
    assert _call(h, "noalloc", p, d, C_na, raw) == 0, lg.library().lin_gemm_last_error(h._h)
    torch.cuda.synchronize()
    h.set_force(None)
    if raw and p.quant == "w8a8_int8":
        _, acc = oracle.linear(p.quant, "none", p.A, p.B, p.sa, p.sb)
        assert np.array_equal(C_na.cpu().numpy(), acc), f"{tag}: int8 accumulators differ"
        assert np.array_equal(C_na.cpu().numpy(), C_ref.cpu().numpy())
        return
    g_na = decode_out(C_na, p.quant)
    g_ref = decode_out(C_ref, p.quant)
    # Same variant, same kernels: bit-identical except the atomic reduction,
    # whose fp32 summation order is not fixed (held to the tolerance instead).
    if force is None or "reduce=atomic" not in force:
        assert np.array_equal(C_na.cpu().numpy(), C_ref.cpu().numpy()), \
            f"{tag}: noalloc and lin_gemm_run outputs differ"
    else:
        assert_close(g_na, g_ref.astype(np.float64), f"{tag}: noalloc vs lin_gemm_run")
    if sampled:
        im, inn = sample_positions(p.M, p.N, 3000, seed=p.M)
        r, _ = reference(p, (im, inn))
        assert_close(g_na[im, inn], r, f"{tag}: noalloc vs oracle")
    else:
        r, _ = reference(p)
        assert_close(g_na, r, f"{tag}: noalloc vs oracle")


def test_block_fp8_pp_split_then_smaller_tile_split(handle):
    # Block FP8 at 512 tokens: ping-pong tiles with K split over scale blocks
    # (32 MiB of partials in the scratch array); then the FP8 decode shape at
    # 64 tokens on split tiles, which overwrites a smaller part of it.
    _check_pair(handle, synth.make(4, 512), sampled=True, tag="first")
    _check_pair(handle, synth.make_custom("fp8_dynamic", "silu", 64, 6144, 4096, seed=5,
                                          bias=True), sampled=True, tag="second")


@pytest.mark.parametrize("reduce", ["lastwg", "atomic", "twopass"])
def test_decode_cross_workgroup_split_twice(handle, reduce):
    # Decode with K split across workgroups: partials and arrival counters in
    # the scratch array; the second call is smaller and its counters must
    # start at zero again.
    spec = f"decode swap=1 split=4 reduce={reduce} waves=8 unroll=2 rows=16"
    big = synth.make_custom("w8a8_int8", "silu", 16, 2048, 4096, seed=3, bias=True)
    small = synth.make_custom("w8a8_int8", "silu", 3, 512, 2048, seed=4, bias=True)
    _check_pair(handle, big, force=spec, raw=True, tag=f"{reduce} first")
    _check_pair(handle, small, force=spec, raw=True, tag=f"{reduce} second")
    fbig = synth.make_custom("fp8_dynamic", "gelu_tanh", 8, 1024, 4096, seed=6, bias=True,
                             residual=True, alpha=0.5)
    fsmall = synth.make_custom("fp8_dynamic", "gelu_tanh", 2, 256, 1024, seed=7, bias=True)
    _check_pair(handle, fbig, force=spec, tag=f"{reduce} fp8 first")
    _check_pair(handle, fsmall, force=spec, tag=f"{reduce} fp8 second")


def test_default_dispatch_decode_and_prefill(handle):
    # Shapes whose variants use no scratch at all pass straight through.
    _check_pair(handle, synth.make(2, 32), tag="fp8 decode 32")
    _check_pair(handle, synth.make(1), tag="tiny bf16")


def test_rejects_partials_beyond_the_scratch(handle):
    # 16 K slices of a 1024 x 24576 fp32 tile grid need 1.5 GiB of partials:
    # rejected on the host before anything is enqueued.
    p = synth.make_custom("fp8_dynamic", "none", 1024, 24576, 4096, seed=1, bias=False)
    handle.set_force("tile bm=128 bn=128 wm=2 wn=2 split=16")
    try:
        d = upload(p)
        C = out_tensor(p)
        rc = _call(handle, "noalloc", p, d, C)
        torch.cuda.synchronize()
        assert rc == UNSUPPORTED
        assert b"static scratch" in lg.library().lin_gemm_last_error(handle._h)
    finally:
        handle.set_force(None)
