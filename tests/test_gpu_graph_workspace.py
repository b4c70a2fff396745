"""A HIP graph captured with a split-K call keeps working after a later call
grows the handle's workspace: the grown-out buffer stays allocated until
the handle is destroyed, so the graph's captured address remains valid."""
import pytest
import torch

import synth
from gpu_util import assert_close, decode_out, reference, upload

lg = pytest.importorskip("epilogue_scaled_gemm_amd")
pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("small_spec,big_spec", [
    ("tile bm=64 bn=128 wm=1 wn=4 split=4", "tile bm=64 bn=128 wm=1 wn=4 split=8"),
    ("decode swap=1 split=4 reduce=twopass waves=8 unroll=2 rows=16",
     "decode swap=1 split=16 reduce=twopass waves=8 unroll=2 rows=16"),
])
def test_captured_graph_survives_workspace_growth(small_spec, big_spec):
    h = lg.Handle()
    try:
        small = synth.make_custom("fp8_dynamic", "silu", 64 if small_spec.startswith("tile") else 8,
                                  1024, 2048, seed=1, bias=True)
        big = synth.make_custom("fp8_dynamic", "none", 256 if big_spec.startswith("tile") else 32,
                                6144, 4096, seed=2)
        ds, db = upload(small), upload(big)
        Cs = torch.empty((small.M, small.N), dtype=torch.int16, device="cuda")
        Cb = torch.empty((big.M, big.N), dtype=torch.int16, device="cuda")

        def call(p, d, C):
            h.run(d["A"], d["B"], C, quant=p.quant, act=p.act, sa=d["sa"], sb=d["sb"],
                  alpha=p.alpha, bias=d["bias"], residual=d["residual"])

        h.set_force(small_spec)
        call(small, ds, Cs)                      # warm: sizes the workspace
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            call(small, ds, Cs)
        h.set_force(big_spec)
        call(big, db, Cb)                        # grows the workspace
        torch.cuda.synchronize()
        ref, _ = reference(small)
        for _ in range(3):
            Cs.fill_(0)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert_close(decode_out(Cs, small.quant), ref, f"replay after growth [{small_spec}]")
        del g
    finally:
        h.set_force(None)
        h.close()


def test_atomic_replay_after_other_split_calls():
    # A graph holding an atomic-reduction decode call, replayed after eager
    # split-K calls (tile and two-pass) have left partials in the same
    # handle workspace: the zero fill travels with the captured call, so
    # every replay still matches the oracle.
    h = lg.Handle()
    try:
        dec = synth.make_custom("fp8_dynamic", "silu", 8, 1024, 4096, seed=5, bias=True)
        til = synth.make_custom("fp8_dynamic", "none", 96, 1024, 4096, seed=6)
        dd, dt = upload(dec), upload(til)
        Cd = torch.empty((dec.M, dec.N), dtype=torch.int16, device="cuda")
        Ct = torch.empty((til.M, til.N), dtype=torch.int16, device="cuda")

        def call(p, d, C):
            h.run(d["A"], d["B"], C, quant=p.quant, act=p.act, sa=d["sa"], sb=d["sb"],
                  alpha=p.alpha, bias=d["bias"], residual=d["residual"])

        # size the workspace for the largest user first, so nothing grows later
        h.set_force("tile bm=64 bn=128 wm=1 wn=4 split=8")
        call(til, dt, Ct)
        atomic = "decode swap=1 split=4 reduce=atomic waves=8 unroll=2 rows=16"
        h.set_force(atomic)
        call(dec, dd, Cd)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            call(dec, dd, Cd)
        ref, _ = reference(dec)
        for spec in ("tile bm=64 bn=128 wm=1 wn=4 split=8",
                     "decode swap=1 split=4 reduce=twopass waves=8 unroll=2 rows=16"):
            h.set_force(spec)
            call(til if spec.startswith("tile") else dec, dt if spec.startswith("tile") else dd,
                 Ct if spec.startswith("tile") else Cd)
            torch.cuda.synchronize()
            Cd.fill_(0)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert_close(decode_out(Cd, dec.quant), ref, f"atomic replay after [{spec}]")
        del g
    finally:
        h.set_force(None)
        h.close()
