"""The grouped (mixture-of-experts) layer against the oracle, through the C
ABI: each expert's segment of rows with its own weight, scales and bias.

Segments of every size class: empty experts, single tokens, segments that
fill one token tile, that spill into a second chunk, that one workgroup
loops over (a max_rows bound, or a mean segment, below the true size) and
that spread over a grid several chunks deep.  int8 is
compared bit-exactly on the raw int32 accumulator; the other modes within
the relative tolerance.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
import synth

lg = pytest.importorskip("epilogue_scaled_gemm_amd")

pytestmark = pytest.mark.gpu


def dev(x):
    if x is None:
        return None
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        x = x.view(np.int16)
    return torch.from_numpy(x).cuda()


def stack(arrs):
    return None if arrs is None or arrs[0] is None else np.ascontiguousarray(np.stack(arrs))


def run(h, g, act=None, raw=False, max_rows=0, alpha=1.0):
    M, N = g["M"], g["N"]
    dt = torch.int32 if (raw and g["quant"] == "w8a8_int8") else (
        torch.float32 if raw else torch.int16)
    C = torch.full((M, N), -1, dtype=dt, device="cuda")
    h.run_grouped(dev(g["A"]), dev(stack(g["Bs"])), C, dev(g["offsets"]), quant=g["quant"],
                  act="raw_acc" if raw else (act or g["act"]), sa=dev(g["sa"]),
                  sb=dev(stack(g["sbs"])), alpha=alpha, bias=dev(stack(g["biases"])),
                  residual=dev(g["residual"]), max_rows=max_rows)
    torch.cuda.synchronize()
    return C.cpu()


def bf16(C, quant):
    t = C.view(torch.float16 if quant == "fp16" else torch.bfloat16)
    return t.double().numpy()


SIZES = {
    "mixed": [3, 0, 1, 16, 0, 17, 5, 2],
    "tiny": [1, 1, 0, 1],
    "wide": [40, 0, 7, 33],
    "deep": [70, 50],   # two 16-token tiles, two chunk slots, three chunks in the first
    # more than 64 experts (two ballot groups), mostly tiny segments
    "many": [int(v) for v in np.random.default_rng(8).choice([0, 0, 1, 2, 3], 100)],
}
# Prefill-sized segments (mean above 32 rows): the grouped tile kernels.
PF_SIZES = {
    "pf_mixed": [100, 0, 37, 300, 5, 64],
    "pf_many": [int(v) for v in np.random.default_rng(9).choice([0, 33, 47, 80, 129], 70)],
}
TILE_SPECS = ["", "tile bm=64 bn=128 wm=1 wn=4", "tile bm=128 bn=128 wm=2 wn=2",
              "tile bm=256 bn=256 wm=2 wn=4"]


# The default grouped variant (no force), its staged form, and the
# eight-wave alternative, staged and not.
SPECS = ["", "decode swap=1 waves=4 unroll=2 rows=32 xs=1",
         "decode swap=1 waves=8 unroll=2 rows=16 xs=0", "decode swap=1 waves=8 unroll=2 rows=16 xs=1"]


@pytest.fixture(scope="module")
def h():
    with lg.Handle() as hh:
        yield hh


@pytest.mark.parametrize("quant,act,N,K", [
    ("bf16", "gelu_tanh", 64, 256),
    ("fp16", "silu", 48, 128),
    ("fp8_dynamic", "silu", 96, 512),
    ("block_fp8", "none", 256, 384),
    ("mxfp4", "gelu_tanh", 80, 512),
])
@pytest.mark.parametrize("sizes", ["mixed", "tiny", "wide", "deep", "many"])
@pytest.mark.parametrize("spec", SPECS)
def test_grouped_matches_oracle(h, quant, act, N, K, sizes, spec):
    g = synth.make_grouped(quant, act, SIZES[sizes], N, K,
                           seed=zlib.crc32(f"{quant}/{sizes}".encode()) % 1000, residual=True)
    h.set_force(spec)
    try:
        got = bf16(run(h, g, alpha=0.75), quant)
    finally:
        h.set_force(None)
    ref, _ = oracle.grouped_linear(quant, act, g["A"], g["Bs"], g["offsets"], sa=g["sa"],
                                   sbs=g["sbs"], biases=g["biases"], residual=g["residual"],
                                   alpha=0.75)
    ok = oracle.within_tolerance(got, ref)
    assert ok.all(), f"{(~ok).sum()} of {ok.size} outside tolerance"


@pytest.mark.parametrize("sizes", ["mixed", "wide", "deep"])
@pytest.mark.parametrize("spec", SPECS)
@pytest.mark.parametrize("max_rows", [0, 1, 16, 33])
def test_grouped_int8_accumulator_bit_exact(h, sizes, spec, max_rows):
    g = synth.make_grouped("w8a8_int8", "silu", SIZES[sizes], 112, 640, seed=5)
    h.set_force(spec)
    try:
        acc = run(h, g, raw=True, max_rows=max_rows).numpy()
        out = bf16(run(h, g, max_rows=max_rows), "w8a8_int8")
    finally:
        h.set_force(None)
    ref, racc = oracle.grouped_linear("w8a8_int8", "silu", g["A"], g["Bs"], g["offsets"],
                                      sa=g["sa"], sbs=g["sbs"], biases=g["biases"])
    assert np.array_equal(acc, racc)
    assert oracle.within_tolerance(out, ref).all()


def test_grouped_uncovered_rows_untouched_and_bad_offsets_clamped(h):
    # offsets not starting at 0, an end beyond M and a decreasing last pair:
    # clamped into [0, M] ([2,6), [6,M), empty); rows outside every segment
    # keep their contents.
    g = synth.make_grouped("fp8_dynamic", "none", [4, 4, 4], 32, 256, seed=9)
    M = g["M"]
    off = np.array([2, 6, 1000, 3], dtype=np.int32)
    C = torch.full((M, 32), 0x1234, dtype=torch.int16, device="cuda")
    h.run_grouped(dev(g["A"]), dev(stack(g["Bs"])), C, dev(off), quant="fp8_dynamic",
                  sa=dev(g["sa"]), sb=dev(stack(g["sbs"])), bias=dev(stack(g["biases"])))
    torch.cuda.synchronize()
    got = bf16(C.cpu(), "fp8_dynamic")
    eff = np.array([2, 6, M, M], dtype=np.int32)
    ref, _ = oracle.grouped_linear("fp8_dynamic", "none", g["A"], g["Bs"], eff, sa=g["sa"],
                                   sbs=g["sbs"], biases=g["biases"])
    assert (C.cpu()[:2] == 0x1234).all()
    assert oracle.within_tolerance(got[2:], ref[2:]).all()


def test_grouped_matches_per_expert_dense_calls(h):
    # The grouped call gives the same bits as lin_gemm_run on each segment
    # with the same variant (four waves, 32 rows, one token tile).
    g = synth.make_grouped("fp8_dynamic", "gelu_tanh", [5, 9, 0, 16], 192, 1024, seed=4)
    h.set_force("decode swap=1 waves=4 unroll=2 rows=32")
    try:
        grp = run(h, g, max_rows=16)
    finally:
        h.set_force(None)
    off = g["offsets"]
    for x in range(4):
        m0, m1 = off[x], off[x + 1]
        if m1 == m0:
            continue
        C = torch.empty((m1 - m0, 192), dtype=torch.int16, device="cuda")
        h.set_force("decode swap=1 split=1 waves=4 unroll=2 rows=32")
        try:
            h.run(dev(g["A"][m0:m1]), dev(g["Bs"][x]), C, quant="fp8_dynamic", act="gelu_tanh",
                  sa=dev(g["sa"][m0:m1]), sb=dev(g["sbs"][x]), bias=dev(g["biases"][x]))
        finally:
            h.set_force(None)
        torch.cuda.synchronize()
        assert torch.equal(C.cpu(), grp[m0:m1])


@pytest.mark.parametrize("quant,act,N,K", [
    ("bf16", "gelu_tanh", 200, 256),
    ("fp16", "none", 128, 136),
    ("fp8_dynamic", "silu", 264, 512),
    ("block_fp8", "gelu_tanh", 256, 384),
    ("mxfp4", "silu", 192, 512),
])
@pytest.mark.parametrize("sizes", list(PF_SIZES))
@pytest.mark.parametrize("spec", TILE_SPECS)
def test_grouped_prefill_matches_oracle(h, quant, act, N, K, sizes, spec):
    g = synth.make_grouped(quant, act, PF_SIZES[sizes], N, K,
                           seed=zlib.crc32(f"pf/{quant}/{sizes}".encode()) % 1000, residual=True)
    h.set_force(spec)
    try:
        got = bf16(run(h, g, alpha=1.5), quant)
    finally:
        h.set_force(None)
    ref, _ = oracle.grouped_linear(quant, act, g["A"], g["Bs"], g["offsets"], sa=g["sa"],
                                   sbs=g["sbs"], biases=g["biases"], residual=g["residual"],
                                   alpha=1.5)
    ok = oracle.within_tolerance(got, ref)
    assert ok.all(), f"{(~ok).sum()} of {ok.size} outside tolerance"


@pytest.mark.parametrize("sizes", list(PF_SIZES))
@pytest.mark.parametrize("spec", TILE_SPECS)
def test_grouped_prefill_int8_bit_exact(h, sizes, spec):
    g = synth.make_grouped("w8a8_int8", "relu", PF_SIZES[sizes], 144, 1040, seed=6)
    h.set_force(spec)
    try:
        acc = run(h, g, raw=True).numpy()
    finally:
        h.set_force(None)
    _, racc = oracle.grouped_linear("w8a8_int8", "relu", g["A"], g["Bs"], g["offsets"],
                                    sa=g["sa"], sbs=g["sbs"])
    assert np.array_equal(acc, racc)


def test_grouped_prefill_rejects_uncompiled_tile(h):
    g = synth.make_grouped("bf16", "none", [40, 40], 64, 64, seed=1)
    h.set_force("tile bm=256 bn=128 wm=2 wn=2")
    try:
        with pytest.raises(lg.LinGemmError):
            run(h, g)
    finally:
        h.set_force(None)


@pytest.mark.parametrize("sizes", ["tiny", "many", "pf_mixed"])
def test_grouped_graph_capture_replays(h, sizes):
    # The grouped call allocates nothing, so it captures without a warm-up;
    # replays with new activations and a new routing copied in between give
    # the eager result bit for bit.
    sz = SIZES.get(sizes) or PF_SIZES[sizes]
    g1 = synth.make_grouped("fp8_dynamic", "silu", sz, 128, 512, seed=21, residual=True)
    g2 = synth.make_grouped("fp8_dynamic", "silu", sz[::-1], 128, 512, seed=22, residual=True)
    B, sb = dev(stack(g1["Bs"])), dev(stack(g1["sbs"]))
    bias = dev(stack(g1["biases"]))
    A, sa, res = dev(g1["A"]), dev(g1["sa"]), dev(g1["residual"])
    off = dev(g1["offsets"])
    C = torch.zeros((g1["M"], 128), dtype=torch.int16, device="cuda")

    def call(out):
        h.run_grouped(A, B, out, off, quant="fp8_dynamic", act="silu", sa=sa, sb=sb, bias=bias,
                      residual=res)

    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        call(C)
    for gg in (g1, g2, g1):
        A.copy_(dev(gg["A"]))
        sa.copy_(dev(gg["sa"]))
        res.copy_(dev(gg["residual"]))
        off.copy_(dev(gg["offsets"]))
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        eager = torch.empty_like(C)
        call(eager)
        torch.cuda.synchronize()
        assert torch.equal(C, eager)


def test_grouped_many_experts_scan():
    # 1000 experts: the expert scan runs over several 256-expert groups
    # (decode path) and the tile scan over many 64-expert groups.
    sizes = [int(v) for v in np.random.default_rng(12).choice([0, 0, 0, 1, 2], 1000)]
    g = synth.make_grouped("fp8_dynamic", "none", sizes, 32, 128, seed=13, bias=True)
    with lg.Handle() as hh:
        for spec in ("", "tile bm=64 bn=128 wm=1 wn=4"):
            hh.set_force(spec)
            try:
                got = bf16(run(hh, g), "fp8_dynamic")
            finally:
                hh.set_force(None)
            ref, _ = oracle.grouped_linear("fp8_dynamic", "none", g["A"], g["Bs"], g["offsets"],
                                           sa=g["sa"], sbs=g["sbs"], biases=g["biases"])
            ok = oracle.within_tolerance(got, ref)
            assert ok.all(), f"[{spec}] {(~ok).sum()} of {ok.size} outside tolerance"
