"""GPU variant invariants: every decode variant (swap-AB on/off, split-K
factors, the three cross-workgroup reductions, wave / unroll shapes), every
compiled tile shape and the ping-pong family (with block-FP8 split-K) gives
the oracle's result; split-K matches the unsplit kernel (int8 bit-exact); the
deterministic reductions are bitwise repeatable; swap-AB equals the direct
orientation."""
import numpy as np
import pytest
import torch

import synth
import oracle
from gpu_util import assert_close, decode_out, reference, run, sample_positions, upload

pytestmark = pytest.mark.gpu

lg = pytest.importorskip("epilogue_scaled_gemm_amd")


@pytest.fixture(scope="module")
def handle():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    h = lg.Handle()
    yield h
    h.set_force(None)
    h.close()


# Every compiled (swap, waves, unroll, rows) combination, with the split-K
# factors and cross-workgroup reductions spread over them.
# (rows = weight rows per workgroup; 8, 12 and 24 leave tile rows masked)
DECODE_SHAPES = [(1, 8, 1, 16), (1, 8, 2, 8), (1, 4, 4, 12), (1, 16, 1, 16), (1, 8, 1, 32),
                 (1, 4, 2, 24), (1, 8, 2, 32), (1, 4, 1, 64), (1, 8, 1, 64), (0, 8, 2, 16),
                 (0, 8, 2, 12), (1, 8, 4, 12), (1, 8, 4, 24), (1, 12, 1, 16), (1, 16, 1, 24),
                 (1, 16, 1, 32), (1, 16, 2, 24)]
SPLITS = [(1, "twopass"), (2, "lastwg"), (4, "atomic"), (8, "twopass"), (16, "lastwg"),
          (4, "twopass"), (2, "atomic")]
DECODE_SPECS = [f"decode swap={sw} split={sp} reduce={rd} waves={w} unroll={u} rows={r}"
                for i, (sw, w, u, r) in enumerate(DECODE_SHAPES)
                for sp, rd in (SPLITS[i % len(SPLITS)], SPLITS[(i + 3) % len(SPLITS)], (1, "twopass"))]

DECODE_PROBLEMS = [
    ("fp8_dynamic", "none", 1, 6144, 4096, True, False),
    ("fp8_dynamic", "gelu_tanh", 5, 1040, 4096, True, True),
    ("w8a8_int8", "silu", 24, 2064, 4096, False, False),
    ("block_fp8", "none", 17, 512, 3072, False, True),
    ("bf16", "silu", 9, 272, 1040, True, True),
    ("fp16", "relu", 32, 144, 528, True, False),
]


@pytest.fixture(scope="module")
def decode_refs():
    out = {}
    for q, a, M, N, K, b, r in DECODE_PROBLEMS:
        p = synth.make_custom(q, a, M, N, K, seed=7 * M + N, bias=b, residual=r)
        ref, _ = reference(p)
        acc = None
        if q == "w8a8_int8":
            _, acc = oracle.linear(q, "none", p.A, p.B, p.sa, p.sb)
        out[(q, M)] = (p, ref, acc)
    return out


@pytest.mark.parametrize("prob", DECODE_PROBLEMS, ids=[f"{p[0]}-M{p[2]}" for p in DECODE_PROBLEMS])
def test_decode_variants_match_oracle(handle, decode_refs, prob):
    p, ref, acc = decode_refs[(prob[0], prob[2])]
    d = upload(p)
    try:
        for spec in DECODE_SPECS:
            rows = int(spec.split("rows=")[1])
            if p.quant == "block_fp8" and 128 % rows:
                with pytest.raises(lg.LinGemmError):
                    handle.set_force(spec)
                    run(handle, p, d)
                continue
            handle.set_force(spec)
            print(f"[variant] {p.name} {spec}", flush=True)
            C = run(handle, p, d)
            assert_close(decode_out(C, p.quant), ref, f"{p.name} [{spec}]")
            if acc is not None:
                Craw = run(handle, p, d, raw=True)
                assert np.array_equal(Craw.cpu().numpy(), acc), f"int8 acc [{spec}]"
    finally:
        handle.set_force(None)


@pytest.mark.parametrize("reduce", ["lastwg", "twopass"])
def test_deterministic_reductions_repeat_bitwise(handle, reduce):
    p = synth.make(2, 16)
    d = upload(p)
    try:
        handle.set_force(f"decode swap=1 split=8 reduce={reduce} waves=8 unroll=1 rows=32")
        first = run(handle, p, d).cpu()
        for _ in range(5):
            assert torch.equal(run(handle, p, d).cpu(), first)
        # and split-K agrees with the unsplit kernel to fp32 reassociation
        handle.set_force("decode swap=1 split=1 reduce=twopass waves=8 unroll=1 rows=32")
        unsplit = decode_out(run(handle, p, d), p.quant)
        assert_close(decode_out(first, p.quant), unsplit, "split vs unsplit")
    finally:
        handle.set_force(None)


@pytest.mark.parametrize("reduce", ["lastwg", "atomic"])
def test_cross_workgroup_arrival_exact_over_repeats(handle, reduce):
    # The last-arrival protocol (partials stored and read at device scope, a
    # wait for the stores' acknowledgement before the arrival increment): int8
    # accumulators are exact whatever the summation order, so any partial
    # that the last workgroup read before it was visible would show up as a
    # wrong value.  Twenty calls, each compared with the oracle exactly.
    p = synth.make(3, 16)
    d = upload(p)
    _, acc = oracle.linear(p.quant, "none", p.A, p.B, p.sa, p.sb)
    try:
        handle.set_force(f"decode swap=1 split=8 reduce={reduce} waves=8 unroll=1 rows=32")
        for i in range(20):
            C = run(handle, p, d, raw=True)
            assert np.array_equal(C.cpu().numpy(), acc), f"{reduce}: call {i} differs"
    finally:
        handle.set_force(None)


def test_swap_ab_equals_direct(handle):
    p = synth.make(3, 8)
    d = upload(p)
    try:
        handle.set_force("decode swap=1 split=1 reduce=twopass waves=8 unroll=2")
        a = run(handle, p, d, raw=True).cpu()
        handle.set_force("decode swap=0 split=1 reduce=twopass waves=8 unroll=2")
        b = run(handle, p, d, raw=True).cpu()
        assert torch.equal(a, b)
    finally:
        handle.set_force(None)


TILE_SPECS = ["tile bm=256 bn=256 wm=2 wn=2", "tile bm=128 bn=256 wm=2 wn=2",
              "tile bm=256 bn=128 wm=2 wn=2", "tile bm=128 bn=128 wm=2 wn=2",
              "tile bm=64 bn=128 wm=1 wn=4", "tile bm=64 bn=64 wm=2 wn=2",
              "tile bm=256 bn=256 wm=2 wn=4", "tile bm=256 bn=128 wm=2 wn=4",
              "tile bm=128 bn=128 wm=2 wn=4",
              # split-K over workgroups (split 8 leaves empty slices on short K)
              "tile bm=64 bn=128 wm=1 wn=4 split=2", "tile bm=128 bn=128 wm=2 wn=2 split=4",
              "tile bm=64 bn=64 wm=2 wn=2 split=8"]
TILE_PROBLEMS = [
    ("bf16", "gelu_tanh", 300, 520, 264, True, True, 0.5),
    ("fp16", "silu", 130, 264, 200, True, False, 1.0),
    ("fp8_dynamic", "relu", 200, 300, 400, True, True, 1.0),
    ("w8a8_int8", "silu", 260, 136, 528, False, False, 1.0),
    ("block_fp8", "none", 270, 512, 384, True, True, 1.0),
    # one and two K stages (pipeline prologue and tail)
    ("bf16", "none", 70, 136, 64, True, False, 1.0),
    ("fp16", "relu", 90, 72, 120, False, True, 1.0),
]


@pytest.mark.parametrize("prob", TILE_PROBLEMS, ids=[f"{p[0]}-K{p[4]}" for p in TILE_PROBLEMS])
def test_tile_shapes_match_oracle(handle, prob):
    q, a, M, N, K, b, r, al = prob
    p = synth.make_custom(q, a, M, N, K, seed=M * 3 + K, bias=b, residual=r, alpha=al)
    ref, _ = reference(p)
    acc = oracle.linear(q, "none", p.A, p.B, p.sa, p.sb)[1] if q == "w8a8_int8" else None
    d = upload(p)
    try:
        for spec in TILE_SPECS:
            handle.set_force(spec)
            print(f"[variant] {p.name} {spec}", flush=True)
            assert_close(decode_out(run(handle, p, d), q), ref, f"{p.name} [{spec}]")
            if acc is not None:
                assert np.array_equal(run(handle, p, d, raw=True).cpu().numpy(), acc), spec
    finally:
        handle.set_force(None)


def test_tile_and_decode_agree_on_small_m(handle):
    # The same M <= 32 problem through both families.
    p = synth.make(4, 32)
    d = upload(p)
    try:
        handle.set_force("tile bm=64 bn=128 wm=1 wn=4")
        t = decode_out(run(handle, p, d), p.quant)
        handle.set_force("decode swap=1 split=4 reduce=lastwg waves=8 unroll=1 rows=64")
        dd = decode_out(run(handle, p, d), p.quant)
        ref, _ = reference(p)
        assert_close(t, ref, "tile")
        assert_close(dd, ref, "decode")
    finally:
        handle.set_force(None)


# Ping-pong family: ragged M / N, K tails inside a 64-byte stage (bf16, fp16,
# int8) and block-FP8 split-K factors (an explicit split above the number of
# scale blocks is clamped; 0 = chosen from the shape).
PP_PROBLEMS = [
    ("bf16", "gelu_tanh", 300, 520, 264, True, True, 0.5, [1]),
    ("fp16", "silu", 130, 264, 200, True, False, 1.0, [1]),
    ("w8a8_int8", "silu", 260, 136, 528, False, False, 1.0, [1]),
    ("block_fp8", "none", 270, 512, 384, True, True, 1.0, [1, 2, 4]),
    ("block_fp8", "gelu_tanh", 600, 1024, 2048, True, False, 1.0, [0, 1, 4, 16]),
    # degenerate sizes: one partial stage, tiles almost empty, one scale block
    ("bf16", "none", 5, 12, 8, True, True, 1.0, [1]),
    ("fp16", "gelu_tanh", 3, 20, 40, False, True, 2.0, [1]),
    ("w8a8_int8", "relu", 17, 40, 16, True, False, 1.0, [1]),
    ("block_fp8", "silu", 3, 128, 128, True, True, 1.0, [1, 2]),
]


@pytest.mark.parametrize("prob", PP_PROBLEMS, ids=[f"{p[0]}-M{p[2]}" for p in PP_PROBLEMS])
def test_pp_variants_match_oracle(handle, prob):
    q, a, M, N, K, b, r, al, splits = prob
    p = synth.make_custom(q, a, M, N, K, seed=M * 5 + N, bias=b, residual=r, alpha=al)
    ref, _ = reference(p)
    acc = oracle.linear(q, "none", p.A, p.B, p.sa, p.sb)[1] if q == "w8a8_int8" else None
    d = upload(p)
    try:
        for sp in splits:
            spec = f"pp split={sp} group=4"
            handle.set_force(spec)
            print(f"[variant] {p.name} {spec} -> {handle.describe(q, M, N, K)}", flush=True)
            assert_close(decode_out(run(handle, p, d), q), ref, f"{p.name} [{spec}]")
            if acc is not None:
                assert np.array_equal(run(handle, p, d, raw=True).cpu().numpy(), acc), spec
    finally:
        handle.set_force(None)


def test_pp_rejects_per_channel_fp8(handle):
    p = synth.make_custom("fp8_dynamic", "none", 64, 256, 512, seed=3, bias=False, residual=False)
    d = upload(p)
    try:
        handle.set_force("pp")
        with pytest.raises(lg.LinGemmError):
            run(handle, p, d)
    finally:
        handle.set_force(None)


@pytest.mark.parametrize("quant,M", [("fp8_dynamic", 128), ("w8a8_int8", 200), ("block_fp8", 64),
                                     ("bf16", 96)])
def test_tile_auto_split_medium_m(handle, quant, M):
    # Medium M with few output tiles: the table's tile variant splits K
    # across workgroups on its own; sampled outputs against the oracle and,
    # for int8, every raw accumulator.
    K = 4096 if quant != "block_fp8" else 12288
    N = 6144 if quant != "block_fp8" else 4096
    p = synth.make_custom(quant, "silu", M, N, K, seed=M + 1, bias=True, residual=True)
    v = handle.describe(quant, M, N, K)
    print(f"[variant] {quant} M={M}: {v}", flush=True)
    assert v.startswith("tile") and "split=" in v
    d = upload(p)
    C = run(handle, p, d)
    im, inn = sample_positions(M, N, 2000, seed=M)
    r, _ = reference(p, (im, inn))
    assert_close(decode_out(C, quant)[im, inn], r, f"{quant} M={M} [{v}]")
    if quant == "w8a8_int8":
        _, acc = oracle.linear_at(quant, "none", p.A, p.B, im, inn, p.sa, p.sb)
        assert np.array_equal(run(handle, p, d, raw=True).cpu().numpy()[im, inn], acc)
